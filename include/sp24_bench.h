/*
 * sp24 measurement support: a dense reference GEMM with the same tiling as the library's token-major sparse
 * GEMM, so that a benchmark can set the sparse kernel's time against a dense one that differs only in what
 * 2:4 sparsity changes. The NVIDIA technical blog on Ampere structured sparsity (Figure 1) and the Orin NN
 * design book (Chapter 7, section 2.1: a 1x4 dot product becomes a 1x2 one) state that gain; this reference
 * isolates it from differences in tiling quality that a vendor dense GEMM would add. Not part of the method:
 * nothing in sp24.h depends on it.
 *
 * Conventions as in sp24.h: caller-owned device pointers, asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream), host-side validation before any HIP call, sp24_status codes, gfx950 only.
 */
#ifndef SP24_BENCH_H
#define SP24_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the dense tiled copy of an M x K bf16 weight: Mp * K * 2, Mp = M rounded up to 16.
 * K must be a positive multiple of 64. Host-only. Errors: SP24_ERR_NULL, SP24_ERR_SHAPE. */
int sp24_bench_dense_tiled_bytes(int64_t M, int64_t K, int64_t* bytes);

/* Copy a dense bf16 weight W (M x K, row pitch ldw elements, ldw * 2 % 16 == 0, 16-byte aligned base) into
 * W_tiled (sp24_bench_dense_tiled_bytes bytes, 16-byte aligned) in the operand order of
 * v_mfma_f32_16x16x32_bf16: tiles of 16 rows x 32 columns (1 KB) stored row block by row block and along K
 * inside a block; byte range [16 l, 16 l + 16) of a tile holds row l % 16, columns 8 (l / 16) .. +7. Rows past M
 * are zero. K must be a multiple of 64. */
int sp24_bench_dense_tile(const void* W, int64_t M, int64_t K, int64_t ldw, void* W_tiled, void* stream);

/* Dense GEMM in the token-major (Linear) layout with fp32 accumulation:
 *   Y[n, m] = sum_k W[m, k] * X[n, k],  X: bf16 N x K (pitch ldx >= K, ldx % 8 == 0), Y: N x M (pitch ldy >= M)
 *   of out_dtype FP32 or BF16 (round to nearest even); W_tiled from sp24_bench_dense_tile.
 * Its kernel has the tiling of sp24_gemm_bf16_ex's token-major kernel for large N: 256 x 256 workgroup tiles
 * in the same persistent order, eight waves of 128 x 64, 32 matrix instructions per wave per stage (here
 * v_mfma_f32_16x16x32_bf16, K advancing 32 per stage), the same barrier placement and epilogue.
 * K a multiple of 64 (below 2^22); 16-byte aligned bases. */
int sp24_bench_gemm_dense_bf16(const void* W_tiled, int64_t M, int64_t K, const void* X, int64_t N, int64_t ldx,
                               void* Y, int out_dtype, int64_t ldy, void* stream);

/* A plain streaming read of `bytes` (a multiple of 16) from src: the achievable floor for a kernel that must read
 * that many bytes once, launch ramp and tail included, against which the few-token GEMMs (bound by streaming
 * their compressed weight) are reported. Every 16-byte word is loaded once; workgroup b writes the XOR of the
 * words it read to sink[b] (16 bytes each; sp24_bench_stream_read_blocks gives the count, so the caller sizes
 * sink and can check that every word was read). 16-byte aligned pointers. */
int sp24_bench_stream_read_blocks(int64_t bytes, int64_t* blocks);
int sp24_bench_stream_read(const void* src, int64_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SP24_BENCH_H */
