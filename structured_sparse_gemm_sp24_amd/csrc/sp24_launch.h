// Host-side launchers of the sp24 kernels (internal to the library; the C ABI in sp24_api.cpp
// validates arguments before calling these).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sp24 {

hipError_t launch_col_norms(const uint16_t* X, int64_t K, int64_t N, int64_t ldx, float* norms, hipStream_t s);

hipError_t launch_prune_compress(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                                 const float* norms, void* values, int val_dtype, uint8_t* meta, hipStream_t s);

hipError_t launch_decompress(const void* values, const uint8_t* meta, int dtype, int64_t M, int64_t K,
                             void* W_out, int64_t ldw, hipStream_t s);

hipError_t launch_gemm_bf16(const uint16_t* values, const uint8_t* meta, int64_t M, int64_t K, const uint16_t* X,
                            int64_t N, int64_t ldx, void* Y, bool out_fp32, int64_t ldy, hipStream_t s);

bool gemm_bf16_skinny_ok(int64_t K, int64_t N, int64_t ldx);
hipError_t launch_gemm_bf16_skinny(const uint16_t* values, const uint8_t* meta, int64_t M, int64_t K, const uint16_t* X,
                                   int64_t N, int64_t ldx, void* Y, bool out_fp32, int64_t ldy, hipStream_t s);

bool gemm_bf16_tiled_ok(int64_t M, int64_t K, int64_t N, int64_t ldx, const void* X);
hipError_t launch_gemm_bf16_tiled(const uint16_t* values, const uint8_t* meta, int64_t M, int64_t K, const uint16_t* X,
                                  int64_t N, int64_t ldx, void* Y, bool out_fp32, int64_t ldy, hipStream_t s);

bool gemm_i8_tiled_ok(int64_t M, int64_t K, int64_t N, int64_t ldx, const void* X);
hipError_t launch_gemm_i8_tiled(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X,
                                int64_t N, int64_t ldx, const float* scale, void* Y, int64_t ldy, hipStream_t s);

hipError_t launch_gemm_i8(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X,
                          int64_t N, int64_t ldx, const float* scale, void* Y, int64_t ldy, hipStream_t s);

}  // namespace sp24
