/*
 * sp24 -- 2:4 fine-grained structured sparsity for Linear and 1x1-conv layers on AMD MI355X (gfx950).
 *
 * The operations follow these pages (cited by title and section):
 *  - Orin NN design book, Chapter 7 "2:4 structured sparsity: benefit conditions and network constraints":
 *    section 2.1 (in every 4 consecutive weights along the input channel K, keep the 2 largest
 *    magnitudes; store only the kept values plus 2-bit positions; at run time the positions select
 *    which activations meet each kept value), section 2.3 and 6.2 (dimensions in multiples of 16,
 *    padding penalties), section 6.1 (a single non-2:4 block silently disables the sparse path on
 *    other stacks -- this library never falls back silently).
 *  - zyxy.net lecture on Wanda 2:4 pruning, section 2.1: score(w_ij) = |w_ij| * ||X_j||_2, the L2 norm
 *    of input channel j's activations over the calibration tokens.
 *  - NVIDIA technical blog on Ampere structured sparsity (Tencent case studies), Figure 1: the
 *    compressed format holds the non-zeros and index metadata; the sparse product does half the
 *    multiplies of the dense one. Its cuSPARSELt section keeps dimensions in multiples of 16 and
 *    picks a plan per input size (here: an internal per-shape kernel choice).
 *  - oeforum post on sparse acceleration: exactly 2 of every 4 are zero, 2-bit metadata per kept
 *    value; int8 and 2:4 combine.
 *
 * Data formats:
 *  W       M x K weight (output channels x input channels), row-major, row pitch ldw elements.
 *  X       K x N activations (input channels x tokens; one NCHW image of a 1x1 conv is Cin x H*W),
 *          row-major, row pitch ldx elements.
 *  Y       M x N output, row-major, row pitch ldy elements.
 *  values, meta -- the compressed weight. Logically, compressed row i holds, for each group g of 4
 *          consecutive columns 4g..4g+3, the two kept elements in ascending column order (kept value
 *          j = 2g + t), and the nibble i0 | (i1 << 2) (0 <= i0 < i1 <= 3, the kept positions) in
 *          metadata byte g/2 of the row, even g in the low nibble. That nibble is the per-value
 *          2-bit index format of gfx950's v_smfmac.
 *          Physically both streams are stored in the order one v_smfmac holds its sparse operand:
 *           - rows are padded to Mp = M rounded up to 16, columns to Kp = K rounded up to
 *             KT = 128 / e dense columns (e = value size in bytes: bf16/fp16 64, fp32 32, int8 128);
 *           - a tile is 16 rows x 64 bytes of values (KT dense columns) and 16 rows x KT/8 bytes of
 *             metadata; tiles are stored row block by row block, along K inside a row block;
 *           - inside a tile each row is cut into 4 quarters (16 bytes of values; KT/32 bytes of
 *             metadata) stored quarter-major: quarter 0 of rows 0..15, then quarter 1, ... -- so for
 *             bf16, byte range [16 l, 16 l + 16) of a values tile and [2 l, 2 l + 2) of its metadata
 *             tile are exactly the A operand and index operand of lane l of one
 *             v_smfmac_f32_16x16x64_bf16 (int8: v_smfmac_i32_16x16x128_i8, 4 metadata bytes);
 *           - byte b of compressed row i is at ((i/16 * Kp/KT + b/T) * 4 + (b%T)/(T/4)) * 4T
 *             + (i%16) * T/4 + b % (T/4), with T = 64 for values and T = KT/8 for metadata;
 *           - padded rows and columns hold value 0 and metadata nibble 0x4 (positions 0 and 1).
 *          Buffer sizes: values Mp * Kp/2 * e bytes, metadata Mp * Kp/8 bytes
 *          (sp24_compressed_bytes computes them).
 *
 * Selection: element t of a group beats element u when its score is larger, or equal with t < u
 * (lower index wins ties); the two elements beaten by at most one other are kept. Scores are |w|
 * (|q| for int8, |-128| = 128) or, for Wanda, the single-precision product fl32(|w|) * norms[j].
 * Inputs must be finite (NaN is outside the contract); norms must be finite and non-negative.
 *
 * Conventions for every entry point:
 *  - All pointers are device pointers owned by the caller; the library allocates nothing and keeps no
 *    per-call state. Every call is asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *  - Arguments are validated on the host before any HIP call; on error nothing is launched and an
 *    sp24_status below is returned. SP24_ERR_HIP reports a launch error (hipGetLastError after the
 *    launch); errors inside a kernel surface at the caller's next synchronisation.
 *  - K must be a positive multiple of 16 (the alignment rule of the pages); M, N >= 1; row pitches
 *    must be at least the row length. M and N need no padding: tails are handled in the kernels.
 *  - Base pointers must be 16-byte aligned, and where stated a row pitch must keep rows 16-byte
 *    aligned (true for any contiguous tensor whose rows are multiples of 16 bytes).
 *  - values/meta passed to sp24_decompress and the GEMMs must be canonical (i0 < i1 in every nibble)
 *    and laid out as above, which sp24_prune_compress always produces; other metadata is outside
 *    the contract. The library cannot check buffer lengths: the caller provides buffers of the
 *    sizes sp24_compressed_bytes reports.
 *  - The device must be gfx950 (MI355X / MI350X), else SP24_ERR_DEVICE.
 *  - Reentrant; concurrent calls on different streams are independent.
 */
#ifndef SP24_H
#define SP24_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SP24_OK = 0,
    SP24_ERR_NULL = -1,   /* a required pointer is NULL */
    SP24_ERR_SHAPE = -2,  /* M, N < 1; K < 16 or K % 16 != 0; a row pitch shorter than the row */
    SP24_ERR_ALIGN = -3,  /* a base pointer or row pitch breaks the stated 16-byte alignment */
    SP24_ERR_DTYPE = -4,  /* unsupported dtype or dtype combination */
    SP24_ERR_ARG = -5,    /* other invalid argument (score mode, norms with magnitude, ...) */
    SP24_ERR_DEVICE = -6, /* no usable device, or the current device is not gfx950 */
    SP24_ERR_HIP = -7     /* the HIP runtime reported an error at launch */
} sp24_status;

typedef enum { SP24_BF16 = 0, SP24_FP16 = 1, SP24_FP32 = 2, SP24_I8 = 3, SP24_I32 = 4 } sp24_dtype;

typedef enum { SP24_SCORE_MAGNITUDE = 0, SP24_SCORE_WANDA = 1 } sp24_score;

/* Operand layout of the *_ex GEMMs:
 *  SP24_FEATURE_MAJOR: X is K x N (input channels x tokens; one NCHW image of a 1x1 conv is
 *                      Cin x H*W), Y is M x N -- the layout of sp24_gemm_bf16 / sp24_gemm_i8.
 *  SP24_TOKEN_MAJOR:   X is N x K (tokens x input channels, the layout of a Linear layer's input),
 *                      Y is N x M; row pitches ldx >= K and ldy >= M. */
typedef enum { SP24_FEATURE_MAJOR = 0, SP24_TOKEN_MAJOR = 1 } sp24_layout;

/* Activation of the fused int8 epilogue: none, or GELU(y) = y/2 (1 + erf(y / sqrt 2)). */
typedef enum { SP24_ACT_NONE = 0, SP24_ACT_GELU = 1 } sp24_activation;

/* Per-input-channel activation norms for Wanda scoring (zyxy.net Wanda lecture, section 2.1).
 *   norms[j] = sqrt( sum_{n<N} X[j*ldx + n]^2 ),  j < K.
 * X: bf16, K x N, any row pitch ldx >= N (16-byte aligned base). norms: fp32[K].
 * The sum of squares is accumulated in double precision, the square root taken in double and
 * rounded once to fp32. K need not be a multiple of 16 here (K >= 1). */
int sp24_col_norms(const void* X, int64_t K, int64_t N, int64_t ldx, float* norms, void* stream);

/* Sizes in bytes of the compressed values and metadata of an M x K weight whose kept values have
 * dtype val_dtype (BF16, FP16, FP32 or I8). Host-only, no HIP call. */
int sp24_compressed_bytes(int64_t M, int64_t K, int val_dtype, int64_t* values_bytes, int64_t* meta_bytes);

/* 2:4 prune and compress (Orin NN design, Chapter 7, section 2.1, Steps 1-2).
 *   W: M x K of dtype in {BF16, FP16, FP32, I8}, pitch ldw with ldw*sizeof(dtype) % 16 == 0.
 *   score: MAGNITUDE (norms must be NULL) or WANDA (norms: fp32[K] device array, dtype not I8).
 *   values: compressed values of val_dtype, where val_dtype == dtype, or BF16 when dtype == FP32 (the
 *           kept fp32 values rounded to nearest even); otherwise kept values are bit-exact copies
 *           (-0 stays -0). meta: the metadata. Both in the tiled layout above, padding included. */
int sp24_prune_compress(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                        const float* norms, void* values, int val_dtype, uint8_t* meta, void* stream);

/* k-of-4 mask (NVIDIA blog on Ampere structured sparsity, progressive sparse training section,
 * Figure 4: the mask first keeps 3 of every 4 weights (25 % sparsity), is recomputed on the remaining
 * weights after tuning to keep 2 of 4 (50 %); the tuning itself is outside this library).
 *   In every group of 4 consecutive columns of a row of W (as sp24_prune_compress: dtype in {BF16, FP16,
 *   FP32, I8}, pitch ldw with ldw*sizeof(dtype) % 16 == 0, MAGNITUDE or WANDA scores, lower index wins
 *   ties), the `keep` elements (1 <= keep <= 4) beaten by fewer than `keep` others are kept.
 *   mask (or NULL): M x K/8 bytes, row-major, the nibble of group g at byte g/2 of its row (even g in
 *     the low nibble), bit t set when position t is kept.
 *   W_out (or NULL; not both NULL): the masked weight, M x K of dtype, pitch ldo with
 *     ldo*sizeof(dtype) % 16 == 0: kept elements bit-copied, +0 at the others.
 * Recomputing a mask on a masked weight with a smaller keep gives the same mask as computing it on the
 * original weight directly (the dropped elements score 0 and lose every comparison). */
int sp24_prune_mask(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int keep, int score,
                    const float* norms, uint8_t* mask, void* W_out, int64_t ldo, void* stream);

/* Input-channel permutation before pruning (Orin NN design, Chapter 7, section 3.1 Step 2 "Channel
 * Permutation" and section 6.3): writes perm (int32[K], device), an order of W's columns in which 2:4
 * pruning keeps at least as much score: permuted column c is original column perm[c]. Prune
 * W[:, perm]; the product is unchanged when X's rows (feature-major; token-major: X's columns) follow
 * perm, which a model usually applies offline to the previous layer's output channels.
 *   Objective: the sum over rows and groups of four of the two largest scores (|w|, or Wanda
 *   fl32(|w|) * norms[original column]), in double precision. Search: `sweeps` sweeps (0..1000) of
 *   round-robin rounds over pairs of groups; each pair moves to the best of its 35 splits into two
 *   groups of four only when that strictly increases its objective, so the objective never decreases
 *   and sweeps = 0 returns the identity. The result is deterministic (the same for any device).
 *   W: M x K of dtype in {BF16, FP16, FP32, I8}, pitch ldw >= K, K a multiple of 4 (at least 8);
 *   score/norms as sp24_prune_compress. Asynchronous: sweeps * (ceil(K/8)*2 - 1) launches on stream. */
int sp24_channel_permutation(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                             const float* norms, int sweeps, int32_t* perm, void* stream);

/* Inverse of the compression: W_out (M x K of dtype in {BF16, FP16, FP32, I8}, pitch ldw with
 * ldw*sizeof(dtype) % 16 == 0) gets every kept value at its original column and +0 (all-zero bits)
 * at the two pruned columns of every group. dtype is the values' dtype. */
int sp24_decompress(const void* values, const uint8_t* meta, int dtype, int64_t M, int64_t K, void* W_out,
                    int64_t ldw, void* stream);

/* Sparse x dense GEMM in bf16 with fp32 accumulation (NVIDIA blog Figure 1; Orin NN design,
 * Chapter 7, section 2.1 Step 3):
 *   Y[m, n] = sum_g sum_{t=0,1} values[m, 2g+t] * X[4g + i_t(m, g), n].
 *   values (bf16) and meta: the compressed M x K weight; X: bf16 K x N (pitch ldx >= N, any value);
 *   Y: M x N (pitch ldy >= N) of out_dtype FP32, or BF16 (the fp32 result rounded to nearest even).
 *   The kernel is chosen from (M, N, K) and the operand alignment; results never depend on it beyond
 *   fp32 summation order. */
int sp24_gemm_bf16(const void* values, const uint8_t* meta, int64_t M, int64_t K, const void* X, int64_t N,
                   int64_t ldx, void* Y, int out_dtype, int64_t ldy, void* stream);

/* Sparse x dense GEMM in int8 with int32 accumulation and per-output-channel dequantization (oeforum
 * post: int8 and 2:4 combine; Orin NN design, Chapter 7, section 3.1 Step 4):
 *   acc[m, n] = sum over kept k of values * X[k, n] (exact int32; |acc| stays below 2^31 for
 *               K <= 262142),
 *   scale != NULL: Y fp32, Y[m, n] = fl32( fl32(acc[m, n]) * scale[m] )  (one multiply, no fusing)
 *   scale == NULL: Y int32, Y[m, n] = acc[m, n].
 *   values (int8) and meta: the compressed M x K weight; X: int8 K x N (pitch ldx >= N); Y pitch
 *   ldy >= N. */
int sp24_gemm_i8(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                 int64_t ldx, const float* scale, void* Y, int64_t ldy, void* stream);

/* The bf16 GEMM for either operand layout and for a batch of products sharing one weight (Orin NN
 * design, Chapter 7, section 2.1: 2:4 sparsity applies to Linear and 1x1-conv layers alike; a 1x1
 * conv over B NCHW images is B feature-major products, a Linear layer's input is token-major):
 *   for b < batch:  Y_b = W_2:4 * X_b  with  X_b = X + b * x_batch_stride,  Y_b = Y + b * y_batch_stride
 *   (strides in elements). layout is an sp24_layout: feature-major X_b is K x N (pitch ldx >= N) and Y_b
 *   M x N (pitch ldy >= N); token-major X_b is N x K (ldx >= K) and Y_b N x M (ldy >= M), i.e.
 *   Y_b[n, m] = sum_g sum_t values[m, 2g+t] * X_b[n, 4g + i_t(m, g)].
 *   batch >= 1. With batch > 1: x_batch_stride >= 0 (entries may overlap or repeat: X is only read),
 *   y_batch_stride at least one Y entry's extent (entries of Y must not overlap), and both strides keep
 *   every entry's base 16-byte aligned; with batch == 1 the strides are ignored. Everything else as
 *   sp24_gemm_bf16, which is this call with batch 1 and SP24_FEATURE_MAJOR. */
int sp24_gemm_bf16_ex(const void* values, const uint8_t* meta, int64_t M, int64_t K, const void* X, int64_t N,
                      int64_t ldx, int64_t x_batch_stride, void* Y, int out_dtype, int64_t ldy, int64_t y_batch_stride,
                      int64_t batch, int layout, void* stream);

/* The int8 GEMM for either operand layout and a batch of products sharing one weight; operands,
 * strides and rules as sp24_gemm_bf16_ex (X int8, Y fp32 with scale or int32 without; the dequant
 * scale is per output channel m in both layouts). sp24_gemm_i8 is this call with batch 1 and
 * SP24_FEATURE_MAJOR. */
int sp24_gemm_i8_ex(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                    int64_t ldx, int64_t x_batch_stride, const float* scale, void* Y, int64_t ldy,
                    int64_t y_batch_stride, int64_t batch, int layout, void* stream);

/* The int8 GEMM with its FFN epilogue fused (NVIDIA blog, quantization section: the sparse int8 BERT
 * of the Sparse-QAT case keeps its FFN in int8 between layers; oeforum post: int8 and 2:4 combine).
 * For every output element, in fp32 with one rounding per step:
 *   y = fl32( fl32(acc[m, n]) * scale[m] );   y = fl32(y + bias[m]) when bias != NULL;
 *   y = GELU(y) = y/2 erfc(-y / sqrt 2) when activation == SP24_ACT_GELU, in fp32 with the rational
 *       erfc approximation of Abramowitz & Stegun (Handbook of Mathematical Functions, formula 7.1.26):
 *       not bit-exact across implementations; |error| <= 8 * 2^-24 * |y| against the exact GELU of the
 *       fp32 input;
 *   stored as out_dtype: SP24_FP32; SP24_BF16 (round to nearest even); or SP24_I8, the requantized code
 *       clamp( rne( fl32(y * inv) ), -127, 127 ) with inv = fl32(1 / out_scale), out_scale > 0 the next
 *       layer's input scale (a multiply by the rounded reciprocal, not a division).
 * scale (fp32[M]) is required; bias is fp32[M] or NULL. Operands, layout, batch and strides as
 * sp24_gemm_i8_ex (Y's element size follows out_dtype). */
int sp24_gemm_i8_fused(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                       int64_t ldx, int64_t x_batch_stride, const float* scale, const float* bias, int activation,
                       void* Y, int out_dtype, float out_scale, int64_t ldy, int64_t y_batch_stride, int64_t batch,
                       int layout, void* stream);

/* Measurement support (no passage of the method: rates are quoted against the MI355X peaks, and this
 * gives the clock those peaks scale with). Launches `blocks` workgroups of 4 waves, one workgroup per
 * compute unit (each takes 96 KB of LDS), in which every wave issues iters x 16 independent
 * v_smfmac_f32_16x16x64_bf16 back to back on register operands, and records for each wave the shader
 * clock cycles (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) of that loop:
 *   out[2 w] = cycles, out[2 w + 1] = real-time ticks, for waves w = 0 .. 4 blocks - 1
 * (device memory owned by the caller, 8 * blocks uint64). Cycles per smfmac = cycles / (16 iters); the
 * sustained shader clock under matrix-core load = cycles / (ticks / 100 MHz). Errors: SP24_ERR_NULL,
 * SP24_ERR_ARG (blocks < 1 or > 65535, iters < 1 or > 10^6). */
int sp24_probe_sclk(int64_t blocks, int iters, uint64_t* out, void* stream);

/* Static description of a status code. */
const char* sp24_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SP24_H */
