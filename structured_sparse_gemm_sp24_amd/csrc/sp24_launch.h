// Host-side launchers of the sp24 kernels (internal to the library; the C ABI in sp24_api.cpp
// validates arguments before calling these).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sp24 {

// Output kinds of the int8 GEMM.
enum OutKind { OUT_I32 = 0, OUT_F32 = 1, OUT_BF16 = 2, OUT_I8 = 3 };

// Operands of one sparse GEMM call, validated by the C ABI. Element strides are in elements of the
// operand's type.
//   feature-major (tm == false): X is K x N (X[k, n] at k * ldx + n), Y is M x N (Y[m, n] at m * ldy + n)
//   token-major   (tm == true):  X is N x K (X[k, n] at n * ldx + k), Y is N x M (Y[m, n] at n * ldy + m)
//   batch b (0 <= b < batch) adds b * sx to X and b * sy to Y; the weight is shared.
struct GemmArgs {
    const void* values;
    const uint8_t* meta;
    int64_t M, K, N;
    const void* X;
    int64_t ldx, sx;
    void* Y;
    int64_t ldy, sy;
    int64_t batch;
    bool tm;
    const float* scale;  // int8 only: per-row dequant scale, or NULL for raw int32 output
    bool out_fp32;       // bf16 only: fp32 output (else bf16)
    // int8 epilogue (with scale): y = fl32(fl32(acc) * scale[m]), + bias[m] when bias is set, GELU when
    // gelu is set, then stored as out_kind (OUT_F32, OUT_BF16 round to nearest even, OUT_I8
    // clamp(rne(fl32(y * inv_scale)), -127, 127)); without scale out_kind is OUT_I32 (raw accumulators)
    const float* bias;
    int gelu;
    int out_kind;
    float inv_scale;
};

hipError_t launch_col_norms(const uint16_t* X, int64_t K, int64_t N, int64_t ldx, float* norms, hipStream_t s);

hipError_t launch_prune_compress(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                                 const float* norms, void* values, int val_dtype, uint8_t* meta, hipStream_t s);

hipError_t launch_prune_mask(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int keep, int score,
                             const float* norms, uint8_t* mask, void* W_out, int64_t ldo, hipStream_t s);

// Shader-clock probe: `blocks` workgroups of 4 waves, cycles and real-time ticks per wave into out.
hipError_t launch_sclk_probe(int64_t blocks, int iters, uint64_t* out, hipStream_t s);
hipError_t launch_channel_permutation(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                                      const float* norms, int sweeps, int32_t* perm, hipStream_t s);

hipError_t launch_decompress(const void* values, const uint8_t* meta, int dtype, int64_t M, int64_t K,
                             void* W_out, int64_t ldw, hipStream_t s);

// bf16 GEMM: the kernel is chosen from the shape, layout and alignment (few tokens, LDS-tiled, direct).
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t s);
bool gemm_bf16_skinny_ok(const GemmArgs& g);
hipError_t launch_gemm_bf16_skinny(const GemmArgs& g, hipStream_t s);
// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();
// Workgroup tile width (256, or 128 for token-major X) of a tiled int8 GEMM launch.
int tiled_tile_width(const GemmArgs& g);
// Few-token GEMM in the Linear layout (token-major, N <= 16) with the weight streamed through LDS.
bool gemm_bf16_fewtok_ok(const GemmArgs& g);
hipError_t launch_gemm_bf16_fewtok(const GemmArgs& g, hipStream_t s);
bool gemm_bf16_tiled_ok(const GemmArgs& g);
hipError_t launch_gemm_bf16_tiled(const GemmArgs& g, hipStream_t s);

// Dense reference with the token-major tiled kernel's tiling (measurement only): the weight converted to the
// MFMA operand order, and the GEMM (token-major X, batch 1; values = the converted weight).
hipError_t launch_dense_tile(const void* W, int64_t M, int64_t K, int64_t ldw, void* Wt, hipStream_t s);
hipError_t launch_gemm_dense_ref(const GemmArgs& g, hipStream_t s);

// Streaming read (measurement only): workgroups used for `bytes`, and the launch.
int stream_read_blocks(int64_t bytes);
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t s);

// int8 GEMM: LDS-tiled when it applies, else direct.
hipError_t launch_gemm_i8(const GemmArgs& g, hipStream_t s);
bool gemm_i8_fewtok_ok(const GemmArgs& g);
hipError_t launch_gemm_i8_fewtok(const GemmArgs& g, hipStream_t s);
bool gemm_i8_tiled_ok(const GemmArgs& g);
hipError_t launch_gemm_i8_tiled(const GemmArgs& g, hipStream_t s);

}  // namespace sp24
