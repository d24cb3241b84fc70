// C ABI of the sp24 library: argument validation (host only, before any HIP call), the device check,
// and dispatch to the kernels. Declarations and the contract live in include/sp24.h.
#include "../../include/sp24.h"
#include "../../include/sp24_bench.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "sp24_launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, -1 = other
std::atomic<int> g_dev_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int elem_size(int dt) {
    switch (dt) {
    case SP24_BF16: case SP24_FP16: return 2;
    case SP24_FP32: case SP24_I32: return 4;
    case SP24_I8: return 1;
    }
    return 0;
}

int check_k(int64_t K) { return (K >= 16 && K % 16 == 0) ? SP24_OK : SP24_ERR_SHAPE; }

// Padded dimensions of the compressed form: rows to 16, columns to 128 / value size.
int64_t padded_m(int64_t M) { return (M + 15) / 16 * 16; }
int64_t padded_k(int64_t K, int vsz) {
    const int64_t kt = 128 / vsz;
    return (K + kt - 1) / kt * kt;
}

// The current device must be gfx950. Cached per device; the first call asks the runtime.
int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return SP24_ERR_DEVICE;
    }
    if (dev < kMaxDevices) {
        int c = g_dev_ok[dev].load(std::memory_order_relaxed);
        if (c != 0) return c > 0 ? SP24_OK : SP24_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return SP24_ERR_DEVICE;
    }
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_dev_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
    return ok ? SP24_OK : SP24_ERR_DEVICE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SP24_OK : SP24_ERR_HIP; }

// Launch-size limits of the kernels (one thread per 16-column chunk, 32-bit chunk counter; the
// direct GEMMs put 64 rows per workgroup in grid.y).
constexpr int64_t kMaxChunks = (int64_t)1 << 32;

// rows * per_row >= kMaxChunks, without forming the product (no signed overflow for any int64 sizes)
bool chunks_exceed(int64_t rows, int64_t per_row) {
    return per_row > 0 && rows > (kMaxChunks - 1) / per_row;
}
constexpr int64_t kMaxRowsDirect = (int64_t)65535 * 64;

}  // namespace

extern "C" {

const char* sp24_status_string(int status) {
    switch (status) {
    case SP24_OK: return "ok";
    case SP24_ERR_NULL: return "a required pointer is NULL";
    case SP24_ERR_SHAPE: return "invalid shape (M, N >= 1; K a positive multiple of 16; pitch >= row length)";
    case SP24_ERR_ALIGN: return "a pointer or row pitch breaks the 16-byte alignment rule";
    case SP24_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case SP24_ERR_ARG: return "invalid argument";
    case SP24_ERR_DEVICE: return "no gfx950 device is current";
    case SP24_ERR_HIP: return "HIP runtime error at launch";
    }
    return "unknown sp24 status";
}

int sp24_compressed_bytes(int64_t M, int64_t K, int val_dtype, int64_t* values_bytes, int64_t* meta_bytes) {
    if (!values_bytes || !meta_bytes) return SP24_ERR_NULL;
    if (val_dtype != SP24_BF16 && val_dtype != SP24_FP16 && val_dtype != SP24_FP32 && val_dtype != SP24_I8)
        return SP24_ERR_DTYPE;
    if (M < 1) return SP24_ERR_SHAPE;
    int st = check_k(K);
    if (st != SP24_OK) return st;
    const int vsz = elem_size(val_dtype);
    const int64_t Mp = padded_m(M), Kp = padded_k(K, vsz);
    *values_bytes = Mp * (Kp / 2) * vsz;
    *meta_bytes = Mp * (Kp / 8);
    return SP24_OK;
}

int sp24_col_norms(const void* X, int64_t K, int64_t N, int64_t ldx, float* norms, void* stream) {
    if (!X || !norms) return SP24_ERR_NULL;
    if (K < 1 || N < 1 || ldx < N) return SP24_ERR_SHAPE;
    if (!aligned16(X)) return SP24_ERR_ALIGN;
    if ((K + 3) / 4 > 0x7FFFFFFF) return SP24_ERR_SHAPE;
    int st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_col_norms(static_cast<const uint16_t*>(X), K, N, ldx, norms,
                                             static_cast<hipStream_t>(stream)));
}

int sp24_prune_compress(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score, const float* norms,
                        void* values, int val_dtype, uint8_t* meta, void* stream) {
    if (!W || !values || !meta) return SP24_ERR_NULL;
    if (dtype != SP24_BF16 && dtype != SP24_FP16 && dtype != SP24_FP32 && dtype != SP24_I8) return SP24_ERR_DTYPE;
    if (!(val_dtype == dtype || (dtype == SP24_FP32 && val_dtype == SP24_BF16))) return SP24_ERR_DTYPE;
    if (score != SP24_SCORE_MAGNITUDE && score != SP24_SCORE_WANDA) return SP24_ERR_ARG;
    if (score == SP24_SCORE_WANDA) {
        if (dtype == SP24_I8) return SP24_ERR_DTYPE;
        if (!norms) return SP24_ERR_NULL;
    } else if (norms) {
        return SP24_ERR_ARG;
    }
    if (M < 1) return SP24_ERR_SHAPE;
    int st = check_k(K);
    if (st != SP24_OK) return st;
    if (ldw < K) return SP24_ERR_SHAPE;
    if (chunks_exceed(padded_m(M), padded_k(K, elem_size(val_dtype)) / 16)) return SP24_ERR_SHAPE;
    const int isz = elem_size(dtype);
    if (!aligned16(W) || !aligned16(values) || !aligned16(meta) || (ldw * isz) % 16 != 0) return SP24_ERR_ALIGN;
    if (norms && !aligned16(norms)) return SP24_ERR_ALIGN;
    st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_prune_compress(W, dtype, M, K, ldw, score, norms, values, val_dtype, meta,
                                                  static_cast<hipStream_t>(stream)));
}

int sp24_prune_mask(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int keep, int score,
                    const float* norms, uint8_t* mask, void* W_out, int64_t ldo, void* stream) {
    if (!W || (!mask && !W_out)) return SP24_ERR_NULL;
    if (dtype != SP24_BF16 && dtype != SP24_FP16 && dtype != SP24_FP32 && dtype != SP24_I8) return SP24_ERR_DTYPE;
    if (keep < 1 || keep > 4) return SP24_ERR_ARG;
    if (score != SP24_SCORE_MAGNITUDE && score != SP24_SCORE_WANDA) return SP24_ERR_ARG;
    if (score == SP24_SCORE_WANDA) {
        if (dtype == SP24_I8) return SP24_ERR_DTYPE;
        if (!norms) return SP24_ERR_NULL;
    } else if (norms) {
        return SP24_ERR_ARG;
    }
    if (M < 1) return SP24_ERR_SHAPE;
    int st = check_k(K);
    if (st != SP24_OK) return st;
    if (ldw < K || (W_out && ldo < K)) return SP24_ERR_SHAPE;
    if (chunks_exceed(M, K / 16)) return SP24_ERR_SHAPE;
    const int isz = elem_size(dtype);
    if (!aligned16(W) || (ldw * isz) % 16 != 0) return SP24_ERR_ALIGN;
    if (mask && !aligned16(mask)) return SP24_ERR_ALIGN;
    if (W_out && (!aligned16(W_out) || (ldo * isz) % 16 != 0)) return SP24_ERR_ALIGN;
    if (norms && !aligned16(norms)) return SP24_ERR_ALIGN;
    st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_prune_mask(W, dtype, M, K, ldw, keep, score, norms, mask, W_out, ldo,
                                              static_cast<hipStream_t>(stream)));
}

int sp24_channel_permutation(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                             const float* norms, int sweeps, int32_t* perm, void* stream) {
    if (!W || !perm) return SP24_ERR_NULL;
    if (dtype != SP24_BF16 && dtype != SP24_FP16 && dtype != SP24_FP32 && dtype != SP24_I8) return SP24_ERR_DTYPE;
    if (score != SP24_SCORE_MAGNITUDE && score != SP24_SCORE_WANDA) return SP24_ERR_ARG;
    if (score == SP24_SCORE_WANDA) {
        if (dtype == SP24_I8) return SP24_ERR_DTYPE;
        if (!norms) return SP24_ERR_NULL;
    } else if (norms) {
        return SP24_ERR_ARG;
    }
    if (sweeps < 0 || sweeps > 1000) return SP24_ERR_ARG;
    if (M < 1 || K < 8 || K % 4 != 0 || ldw < K || K > ((int64_t)1 << 30)) return SP24_ERR_SHAPE;
    const int isz = elem_size(dtype);
    if ((reinterpret_cast<uintptr_t>(W) % isz) != 0 || (reinterpret_cast<uintptr_t>(perm) & 3) != 0) return SP24_ERR_ALIGN;
    if (norms && (reinterpret_cast<uintptr_t>(norms) & 3) != 0) return SP24_ERR_ALIGN;
    const int st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_channel_permutation(W, dtype, M, K, ldw, score, norms, sweeps, perm,
                                                       static_cast<hipStream_t>(stream)));
}

int sp24_decompress(const void* values, const uint8_t* meta, int dtype, int64_t M, int64_t K, void* W_out, int64_t ldw,
                    void* stream) {
    if (!values || !meta || !W_out) return SP24_ERR_NULL;
    if (dtype != SP24_BF16 && dtype != SP24_FP16 && dtype != SP24_FP32 && dtype != SP24_I8) return SP24_ERR_DTYPE;
    if (M < 1) return SP24_ERR_SHAPE;
    int st = check_k(K);
    if (st != SP24_OK) return st;
    if (ldw < K) return SP24_ERR_SHAPE;
    if (chunks_exceed(padded_m(M), padded_k(K, elem_size(dtype)) / 16)) return SP24_ERR_SHAPE;  // one thread per padded chunk
    const int isz = elem_size(dtype);
    if (!aligned16(values) || !aligned16(meta) || !aligned16(W_out) || (ldw * isz) % 16 != 0) return SP24_ERR_ALIGN;
    st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(
        sp24::launch_decompress(values, meta, dtype, M, K, W_out, ldw, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared validation of the GEMM operands (both dtypes); fills g on success. esx / esy: element sizes
// of X and Y.
int check_gemm(const void* values, const uint8_t* meta, int64_t M, int64_t K, const void* X, int64_t N, int64_t ldx,
               int64_t sx, void* Y, int64_t ldy, int64_t sy, int64_t batch, int layout, int esx, int esy,
               sp24::GemmArgs& g) {
    if (!values || !meta || !X || !Y) return SP24_ERR_NULL;
    if (layout != SP24_FEATURE_MAJOR && layout != SP24_TOKEN_MAJOR) return SP24_ERR_ARG;
    if (M < 1 || N < 1 || batch < 1) return SP24_ERR_SHAPE;
    int st = check_k(K);
    if (st != SP24_OK) return st;
    const bool tm = layout == SP24_TOKEN_MAJOR;
    // X rows hold N (feature-major) or K (token-major) elements, Y rows N or M
    if (ldx < (tm ? K : N) || ldy < (tm ? M : N)) return SP24_ERR_SHAPE;
    if (M > kMaxRowsDirect || N > ((int64_t)1 << 31)) return SP24_ERR_SHAPE;
    if (batch > 1) {
        // batch entries of Y must not overlap (X may: it is only read)
        const int64_t y_extent = tm ? (N - 1) * ldy + M : (M - 1) * ldy + N;
        if (sx < 0 || sy < y_extent) return SP24_ERR_SHAPE;
        if ((sx * esx) % 16 != 0 || (sy * esy) % 16 != 0) return SP24_ERR_ALIGN;
    }
    if (!aligned16(values) || !aligned16(meta) || !aligned16(X) || !aligned16(Y)) return SP24_ERR_ALIGN;
    g.values = values;
    g.meta = meta;
    g.M = M; g.K = K; g.N = N;
    g.X = X; g.ldx = ldx; g.sx = batch > 1 ? sx : 0;
    g.Y = Y; g.ldy = ldy; g.sy = batch > 1 ? sy : 0;
    g.batch = batch;
    g.tm = tm;
    g.scale = nullptr;
    g.out_fp32 = false;
    g.bias = nullptr;
    g.gelu = 0;
    g.out_kind = sp24::OUT_I32;
    g.inv_scale = 1.f;
    return SP24_OK;
}

}  // namespace

extern "C" {

int sp24_gemm_bf16_ex(const void* values, const uint8_t* meta, int64_t M, int64_t K, const void* X, int64_t N,
                      int64_t ldx, int64_t x_batch_stride, void* Y, int out_dtype, int64_t ldy, int64_t y_batch_stride,
                      int64_t batch, int layout, void* stream) {
    if (out_dtype != SP24_FP32 && out_dtype != SP24_BF16) {
        if (!values || !meta || !X || !Y) return SP24_ERR_NULL;
        return SP24_ERR_DTYPE;
    }
    sp24::GemmArgs g;
    int st = check_gemm(values, meta, M, K, X, N, ldx, x_batch_stride, Y, ldy, y_batch_stride, batch, layout, 2,
                        out_dtype == SP24_FP32 ? 4 : 2, g);
    if (st != SP24_OK) return st;
    g.out_fp32 = out_dtype == SP24_FP32;
    st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_gemm_bf16(g, static_cast<hipStream_t>(stream)));
}

int sp24_gemm_bf16(const void* values, const uint8_t* meta, int64_t M, int64_t K, const void* X, int64_t N,
                   int64_t ldx, void* Y, int out_dtype, int64_t ldy, void* stream) {
    return sp24_gemm_bf16_ex(values, meta, M, K, X, N, ldx, 0, Y, out_dtype, ldy, 0, 1, SP24_FEATURE_MAJOR, stream);
}

int sp24_gemm_i8_ex(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                    int64_t ldx, int64_t x_batch_stride, const float* scale, void* Y, int64_t ldy,
                    int64_t y_batch_stride, int64_t batch, int layout, void* stream) {
    sp24::GemmArgs g;
    int st = check_gemm(values, meta, M, K, X, N, ldx, x_batch_stride, Y, ldy, y_batch_stride, batch, layout, 1, 4, g);
    if (st != SP24_OK) return st;
    if (K > 262142) return SP24_ERR_SHAPE;  // keeps |acc| < 2^31 for any int8 inputs
    if (scale && (reinterpret_cast<uintptr_t>(scale) & 3) != 0) return SP24_ERR_ALIGN;
    g.scale = scale;
    g.out_kind = scale ? sp24::OUT_F32 : sp24::OUT_I32;
    st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_gemm_i8(g, static_cast<hipStream_t>(stream)));
}

int sp24_gemm_i8_fused(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                       int64_t ldx, int64_t x_batch_stride, const float* scale, const float* bias, int activation,
                       void* Y, int out_dtype, float out_scale, int64_t ldy, int64_t y_batch_stride, int64_t batch,
                       int layout, void* stream) {
    if (!scale) return SP24_ERR_NULL;
    if (out_dtype != SP24_FP32 && out_dtype != SP24_BF16 && out_dtype != SP24_I8) {
        if (!values || !meta || !X || !Y) return SP24_ERR_NULL;
        return SP24_ERR_DTYPE;
    }
    const int es = out_dtype == SP24_FP32 ? 4 : (out_dtype == SP24_BF16 ? 2 : 1);
    sp24::GemmArgs g;
    int st = check_gemm(values, meta, M, K, X, N, ldx, x_batch_stride, Y, ldy, y_batch_stride, batch, layout, 1, es, g);
    if (st != SP24_OK) return st;
    if (K > 262142) return SP24_ERR_SHAPE;  // keeps |acc| < 2^31 for any int8 inputs
    if (activation != SP24_ACT_NONE && activation != SP24_ACT_GELU) return SP24_ERR_ARG;
    if (out_dtype == SP24_I8 && !(out_scale > 0.f && out_scale < 3.4e38f)) return SP24_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(scale) & 3) != 0 || (bias && (reinterpret_cast<uintptr_t>(bias) & 3) != 0))
        return SP24_ERR_ALIGN;
    g.scale = scale;
    g.bias = bias;
    g.gelu = activation == SP24_ACT_GELU;
    g.out_kind = out_dtype == SP24_FP32 ? sp24::OUT_F32 : (out_dtype == SP24_BF16 ? sp24::OUT_BF16 : sp24::OUT_I8);
    g.inv_scale = 1.0f / out_scale;  // IEEE single division, rounded once
    st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_gemm_i8(g, static_cast<hipStream_t>(stream)));
}

int sp24_gemm_i8(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                 int64_t ldx, const float* scale, void* Y, int64_t ldy, void* stream) {
    return sp24_gemm_i8_ex(values, meta, M, K, X, N, ldx, 0, scale, Y, ldy, 0, 1, SP24_FEATURE_MAJOR, stream);
}

int sp24_probe_sclk(int64_t blocks, int iters, uint64_t* out, void* stream) {
    if (!out) return SP24_ERR_NULL;
    if (blocks < 1 || blocks > 65535 || iters < 1 || iters > 1000000) return SP24_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(out) & 7) != 0) return SP24_ERR_ALIGN;
    const int st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_sclk_probe(blocks, iters, out, static_cast<hipStream_t>(stream)));
}


/* ---- measurement support: the dense reference with the token-major tiled kernel's tiling ---- */

int sp24_bench_dense_tiled_bytes(int64_t M, int64_t K, int64_t* bytes) {
    if (!bytes) return SP24_ERR_NULL;
    if (M < 1 || K < 64 || K % 64 != 0) return SP24_ERR_SHAPE;
    *bytes = padded_m(M) * K * 2;
    return SP24_OK;
}

int sp24_bench_dense_tile(const void* W, int64_t M, int64_t K, int64_t ldw, void* W_tiled, void* stream) {
    if (!W || !W_tiled) return SP24_ERR_NULL;
    if (M < 1 || K < 64 || K % 64 != 0 || ldw < K) return SP24_ERR_SHAPE;
    if (!aligned16(W) || !aligned16(W_tiled) || (ldw * 2) % 16 != 0) return SP24_ERR_ALIGN;
    if (chunks_exceed(padded_m(M) / 16, (K / 32) * 64)) return SP24_ERR_SHAPE;
    const int st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_dense_tile(W, M, K, ldw, W_tiled, static_cast<hipStream_t>(stream)));
}

int sp24_bench_gemm_dense_bf16(const void* W_tiled, int64_t M, int64_t K, const void* X, int64_t N, int64_t ldx, void* Y,
                               int out_dtype, int64_t ldy, void* stream) {
    if (!W_tiled || !X || !Y) return SP24_ERR_NULL;
    if (out_dtype != SP24_FP32 && out_dtype != SP24_BF16) return SP24_ERR_DTYPE;
    if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || ldx < K || ldy < M) return SP24_ERR_SHAPE;
    if (K >= ((int64_t)1 << 22) || ldx >= ((int64_t)1 << 22) || ldy >= ((int64_t)1 << 31)) return SP24_ERR_SHAPE;
    if (((M + 255) / 256) * ((N + 255) / 256) >= ((int64_t)1 << 30)) return SP24_ERR_SHAPE;
    if (!aligned16(W_tiled) || !aligned16(X) || ldx % 8 != 0 || !aligned16(Y)) return SP24_ERR_ALIGN;
    const int st = check_device();
    if (st != SP24_OK) return st;
    sp24::GemmArgs g = {};
    g.values = W_tiled;
    g.meta = nullptr;
    g.M = M; g.K = K; g.N = N;
    g.X = X; g.ldx = ldx; g.sx = 0;
    g.Y = Y; g.ldy = ldy; g.sy = 0;
    g.batch = 1;
    g.tm = true;
    g.out_fp32 = out_dtype == SP24_FP32;
    return hip_status(sp24::launch_gemm_dense_ref(g, static_cast<hipStream_t>(stream)));
}

int sp24_bench_stream_read_blocks(int64_t bytes, int64_t* blocks) {
    if (!blocks) return SP24_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0) return SP24_ERR_SHAPE;
    const int st = check_device();
    if (st != SP24_OK) return st;
    *blocks = sp24::stream_read_blocks(bytes);
    return SP24_OK;
}

int sp24_bench_stream_read(const void* src, int64_t bytes, void* sink, void* stream) {
    if (!src || !sink) return SP24_ERR_NULL;
    if (bytes < 16 || bytes % 16 != 0) return SP24_ERR_SHAPE;
    if (!aligned16(src) || !aligned16(sink)) return SP24_ERR_ALIGN;
    const int st = check_device();
    if (st != SP24_OK) return st;
    return hip_status(sp24::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}
}  // extern "C"
