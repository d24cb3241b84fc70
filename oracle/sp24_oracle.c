/*
 * sp24 CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the 2:4 structured-sparse path computes.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load it. The product
 * library never links or calls it, and this file shares no code, header, table or helper with
 * the HIP kernels.
 *
 * Sources (the pages are cited by title and section; they are the authority on what is computed):
 *  [ORIN7]  "Chapter 7: 2:4 structured sparsity: benefit conditions and network constraints" (Orin NN
 *           design book), section 2.1 hardware execution flow (Step 1 prune, Step 2 compressed storage
 *           of values plus 2-bit metadata, Step 3 metadata mux feeding the ALU), section 2.3 alignment,
 *           section 5 exercise Q1, section 6.1 ("ghost sparsity" check that every 1x4 block has 2 zeros).
 *  [NVBLOG] NVIDIA technical blog (zhidx mirror) on Ampere fine-grained structured sparsity with
 *           Tencent case studies: Figure 1 (2:4 pattern; only non-zeros and index metadata stored),
 *           the quantization section (scale chosen to cover 99.99 % of values).
 *  [WANDA]  zyxy.net lecture "Wanda: 2:4 sparse inference without retraining", section 2.1 (score =
 *           |w| times the L2 norm of the input activation channel).
 *  [FORUM]  oeforum post on sparse acceleration: exactly 2 of every 4 consecutive weights are zero;
 *           2-bit metadata per kept value; the multiply only takes the matching activations.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - groups are 4 consecutive weights along K inside one row of the M x K weight [ORIN7 2.1];
 *  - exactly two slots are kept per group; between equal scores the lower index wins;
 *  - kept values are stored in ascending position order [ORIN7 2.1 Step 2 shows [-0.5, 0.2] for
 *    positions 1 and 3];
 *  - metadata nibble of group g = i0 | (i1 << 2) with i0 < i1, group g of a row in byte g/2 of that
 *    row's metadata bytes, even g in the low nibble; the bytes of both streams are placed in 16-row
 *    tiles in the order of the sparse MFMA operand (see "compressed layout" below);
 *  - the Wanda score is the single-precision product fl32(|w|) * norms[j]; norms are an input;
 *  - the pruned slots decompress to +0.
 *
 * Precision: scores are compared in double (|w| of bf16/fp16/fp32 is exact in double); norms and
 * the bf16 GEMM accumulate in double; the int8 GEMM accumulates exactly in int64 and applies the
 * dequant as fl32(fl32(acc) * scale[m]). Build with -ffp-contract=off and no fast-math.
 * OpenMP over independent rows is only for timing; results do not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_BF16 = 0, OR_FP16 = 1, OR_FP32 = 2, OR_I8 = 3, OR_I32 = 4 };
enum { OR_MAGNITUDE = 0, OR_WANDA = 1 };
enum { OR_OK = 0, OR_EARG = -1, OR_EMETA = -2, OR_EOVERFLOW = -3 };

/* ---------------------------------------------------------------- number formats (definitions) */

/* bf16 is the upper half of an IEEE binary32 word, so its value is that word's value. */
static double bf16_value(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double fp16_value(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-10 * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sign ? -v : v;
}

static double fp32_value(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Value of a bf16 pattern for rounding purposes: the pattern just above the largest finite one
 * stands for 2^128, the value the next step would have with an unbounded exponent (IEEE 754
 * rounds as if the exponent range were unbounded, then overflows to infinity). */
static double bf16_value_unbounded(uint32_t h) {
    if ((h & 0x7FFF) == 0x7F80) return (h & 0x8000) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
    return bf16_value((uint16_t)h);
}

/* fp32 -> bf16, round to nearest, ties to even, written from the definition: the two bf16
 * neighbours of x are the truncation t (toward zero) and the next pattern t+1 (away from zero);
 * pick the nearer; on a tie pick the one with an even last bit. Finite input, or infinity. */
static uint16_t fp32_to_bf16_rne(uint32_t u) {
    uint32_t t = u >> 16;
    if ((u & 0xFFFF) == 0) return (uint16_t)t; /* exactly representable (also +-0, +-inf) */
    double x = fp32_value(u);
    double lo = bf16_value((uint16_t)t);
    double hi = bf16_value_unbounded(t + 1);
    double dlo = fabs(x - lo), dhi = fabs(hi - x);
    if (dlo < dhi) return (uint16_t)t;
    if (dhi < dlo) return (uint16_t)(t + 1);
    return (t & 1) ? (uint16_t)(t + 1) : (uint16_t)t;
}

static size_t dtype_size(int dt) {
    switch (dt) {
    case OR_BF16: case OR_FP16: return 2;
    case OR_FP32: case OR_I32: return 4;
    case OR_I8: return 1;
    }
    return 0;
}

/* Exact value of element idx of a buffer of the given dtype. */
static double elem_value(const void* p, int dt, size_t idx) {
    switch (dt) {
    case OR_BF16: return bf16_value(((const uint16_t*)p)[idx]);
    case OR_FP16: return fp16_value(((const uint16_t*)p)[idx]);
    case OR_FP32: return fp32_value(((const uint32_t*)p)[idx]);
    case OR_I8: return (double)((const int8_t*)p)[idx];
    }
    return NAN;
}

/* ---------------------------------------------------------------- sp24 column norms [WANDA 2.1] */

/* norms[j] = sqrt(sum_n X[j, n]^2) over the N calibration tokens of input channel j. X is bf16,
 * K x N row-major with row pitch ldx. Squares and the sum are taken in double, in index order,
 * then the square root is rounded once to fp32. */
int oracle_col_norms(const uint16_t* X, int64_t K, int64_t N, int64_t ldx, float* norms) {
    if (!X || !norms || K < 0 || N < 0 || ldx < N) return OR_EARG;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; j++) {
        double s = 0.0;
        for (int64_t n = 0; n < N; n++) {
            double x = bf16_value(X[j * ldx + n]);
            s += x * x;
        }
        norms[j] = (float)sqrt(s);
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- compressed layout */

/* Where the compressed stream lives in memory. The pages fix what is stored (the kept values in
 * ascending position order plus 2 bits of position each [ORIN7 2.1 Step 2; NVBLOG Figure 1]) but
 * not the placement; this library stores it in the order gfx950's sparse MFMA holds its sparse
 * operand, so a tile can be copied straight into the instruction's registers:
 *  - rows are padded to Mp = M rounded up to 16, columns to Kp = K rounded up to KT = 128 / e
 *    dense columns (e = value size in bytes: bf16/fp16 64, fp32 32, int8 128);
 *  - a tile is 16 rows x 64 bytes of values (= KT dense columns) and 16 rows x KT/8 bytes of
 *    metadata; tiles go row-block by row-block, and along K inside a row block;
 *  - inside a tile each row's bytes are cut into 4 quarters (16 bytes of values, KT/32 bytes of
 *    metadata) and stored quarter-major: quarter 0 of rows 0..15, then quarter 1, ...;
 *  - padding holds value 0 and metadata nibble 0x4 (positions 0 and 1).
 * The offset functions below are that definition written out. */

static int64_t dense_tile_width(int esize) { return 128 / esize; }

static int64_t padded_k(int64_t K, int esize) {
    int64_t kt = dense_tile_width(esize);
    return (K + kt - 1) / kt * kt;
}

static int64_t padded_m(int64_t M) { return (M + 15) / 16 * 16; }

/* Byte offset of byte b (0 <= b < Kp*e/2) of compressed row i in the values buffer. */
static size_t values_offset(int64_t i, int64_t b, int64_t K, int esize) {
    const int64_t tiles_per_row = padded_k(K, esize) / dense_tile_width(esize);
    const int64_t rb = i / 16, r = i % 16;
    const int64_t t = b / 64, c = (b % 64) / 16, o = b % 16;
    return (size_t)(((rb * tiles_per_row + t) * 4 + c) * 256 + r * 16 + o);
}

/* Byte offset of metadata byte mb (0 <= mb < Kp/8) of row i in the metadata buffer. */
static size_t meta_offset(int64_t i, int64_t mb, int64_t K, int esize) {
    const int64_t tiles_per_row = padded_k(K, esize) / dense_tile_width(esize);
    const int64_t tm = dense_tile_width(esize) / 8, qm = tm / 4;
    const int64_t rb = i / 16, r = i % 16;
    const int64_t t = mb / tm, c = (mb % tm) / qm, o = mb % qm;
    return (size_t)(((rb * tiles_per_row + t) * 4 + c) * (16 * qm) + r * qm + o);
}

/* Sizes of the two buffers for an M x K weight of the given value dtype. */
int oracle_compressed_bytes(int64_t M, int64_t K, int val_dtype, int64_t* values_bytes, int64_t* meta_bytes) {
    const int esize = (int)dtype_size(val_dtype);
    if (esize == 0 || val_dtype == OR_I32 || M < 0 || K < 0) return OR_EARG;
    *values_bytes = padded_m(M) * padded_k(K, esize) / 2 * esize;
    *meta_bytes = padded_m(M) * padded_k(K, esize) / 8;
    return OR_OK;
}

int64_t oracle_values_offset(int64_t i, int64_t b, int64_t K, int esize) { return (int64_t)values_offset(i, b, K, esize); }
int64_t oracle_meta_offset(int64_t i, int64_t mb, int64_t K, int esize) { return (int64_t)meta_offset(i, mb, K, esize); }

/* Nibble (kept positions) of group g of row i. */
static int get_nibble(const uint8_t* meta, int64_t i, int64_t g, int64_t K, int esize) {
    return (meta[meta_offset(i, g / 2, K, esize)] >> (4 * (g % 2))) & 0xF;
}

/* ---------------------------------------------------------------- prune + compress [ORIN7 2.1] */

/* Scores of one group of four: magnitude |w| [ORIN7 2.1 Step 1] or Wanda fl32(|w|) * norm_j
 * [WANDA 2.1]. */
static void group_scores(const void* W, int dtype, size_t base, int score, const float* norms, int64_t k0,
                         double s[4]) {
    for (int t = 0; t < 4; t++) {
        double a = fabs(elem_value(W, dtype, base + (size_t)t));
        if (score == OR_WANDA) {
            float af = (float)a;            /* exact: |w| of bf16/fp16/fp32 is an fp32 value */
            float prod = af * norms[k0 + t]; /* one IEEE single-precision multiply */
            s[t] = (double)prod;
        } else {
            s[t] = a;
        }
    }
}

/* The two kept positions of a group: element t is kept when at most one other element beats it,
 * where u beats t if its score is larger, or equal with a lower index. Returns i0 < i1. */
static void keep_two(const double s[4], int* i0, int* i1) {
    int kept[2], nk = 0;
    for (int t = 0; t < 4; t++) {
        int beaten_by = 0;
        for (int u = 0; u < 4; u++) {
            if (u == t) continue;
            if (s[u] > s[t] || (s[u] == s[t] && u < t)) beaten_by++;
        }
        if (beaten_by <= 1) kept[nk++] = t;
    }
    /* a strict total order always leaves exactly two elements beaten by at most one other */
    *i0 = kept[0];
    *i1 = kept[1];
}

/* W: M x K row-major (pitch ldw elements) of dtype in {BF16, FP16, FP32, I8}, K % 16 == 0.
 * Writes the compressed values (val_dtype) and metadata in the layout above; the buffers must hold
 * oracle_compressed_bytes(M, K, val_dtype) bytes. val_dtype equals dtype, or is BF16 when dtype is
 * FP32 (round to nearest even). score WANDA needs norms[K] and a float dtype. */
int oracle_prune_compress(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                          const float* norms, void* values, int val_dtype, uint8_t* meta) {
    if (!W || !values || !meta || M < 0 || K < 0 || K % 16 != 0 || ldw < K) return OR_EARG;
    if (dtype != OR_BF16 && dtype != OR_FP16 && dtype != OR_FP32 && dtype != OR_I8) return OR_EARG;
    if (!(val_dtype == dtype || (dtype == OR_FP32 && val_dtype == OR_BF16))) return OR_EARG;
    if (score == OR_WANDA && (!norms || dtype == OR_I8)) return OR_EARG;
    if (score != OR_WANDA && score != OR_MAGNITUDE) return OR_EARG;
    const size_t isz = dtype_size(dtype);
    const int vsz = (int)dtype_size(val_dtype);
    int64_t vbytes, mbytes;
    oracle_compressed_bytes(M, K, val_dtype, &vbytes, &mbytes);
    memset(values, 0, (size_t)vbytes);          /* padding: value 0 */
    memset(meta, 0x44, (size_t)mbytes);          /* padding: positions 0 and 1 */
    const int64_t G = K / 4;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        for (int64_t g = 0; g < G; g++) {
            size_t base = (size_t)i * (size_t)ldw + (size_t)(4 * g);
            double s[4];
            int i0, i1;
            group_scores(W, dtype, base, score, norms, 4 * g, s);
            keep_two(s, &i0, &i1);
            int pos[2] = {i0, i1};
            for (int t = 0; t < 2; t++) {
                size_t src = base + (size_t)pos[t];
                int64_t j = 2 * g + t; /* index of the kept value in the compressed row */
                char* dst = (char*)values + values_offset(i, j * vsz, K, vsz);
                if (val_dtype == dtype) {
                    memcpy(dst, (const char*)W + src * isz, isz); /* bit copy */
                } else {
                    uint32_t u;
                    memcpy(&u, (const char*)W + src * 4, 4);
                    uint16_t h = fp32_to_bf16_rne(u);
                    memcpy(dst, &h, 2);
                }
            }
            uint8_t nib = (uint8_t)(i0 | (i1 << 2));
            uint8_t* mb = meta + meta_offset(i, g / 2, K, vsz);
            *mb = (uint8_t)((*mb & (0xF0 >> (4 * (g % 2)))) | (nib << (4 * (g % 2))));
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- k-of-4 masks [NVBLOG progressive] */

/* NVIDIA blog on Ampere structured sparsity, progressive sparse training section, Figure 4: the mask
 * first keeps 3 of every 4 weights (25 % sparsity), later 2 of 4 (50 %). Element t of a group is kept
 * when fewer than `keep` other elements beat it (u beats t if its score is larger, or equal with a lower
 * index -- the rule of keep_two). Returns the mask nibble, bit t set when t is kept. */
static int keep_mask(const double s[4], int keep) {
    int nib = 0;
    for (int t = 0; t < 4; t++) {
        int beaten_by = 0;
        for (int u = 0; u < 4; u++) {
            if (u == t) continue;
            if (s[u] > s[t] || (s[u] == s[t] && u < t)) beaten_by++;
        }
        if (beaten_by < keep) nib |= 1 << t;
    }
    return nib;
}

/* W: M x K (pitch ldw) of dtype in {BF16, FP16, FP32, I8}, K % 16 == 0, 1 <= keep <= 4. mask (or NULL):
 * M x K/8 bytes, row-major, the nibble of group g at byte g/2 (even g low). W_out (or NULL): M x K
 * (pitch ldo) with the kept elements bit-copied and +0 elsewhere. */
int oracle_prune_mask(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int keep, int score,
                      const float* norms, uint8_t* mask, void* W_out, int64_t ldo) {
    if (!W || (!mask && !W_out) || M < 0 || K < 0 || K % 16 != 0 || ldw < K || keep < 1 || keep > 4)
        return OR_EARG;
    if (W_out && ldo < K) return OR_EARG;
    if (dtype != OR_BF16 && dtype != OR_FP16 && dtype != OR_FP32 && dtype != OR_I8) return OR_EARG;
    if (score == OR_WANDA && (!norms || dtype == OR_I8)) return OR_EARG;
    if (score != OR_WANDA && score != OR_MAGNITUDE) return OR_EARG;
    const size_t isz = dtype_size(dtype);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        for (int64_t g = 0; g < K / 4; g++) {
            size_t base = (size_t)i * (size_t)ldw + (size_t)(4 * g);
            double s[4];
            group_scores(W, dtype, base, score, norms, 4 * g, s);
            int nib = keep_mask(s, keep);
            if (mask) {
                uint8_t* mb = mask + (size_t)i * (size_t)(K / 8) + (size_t)(g / 2);
                *mb = (uint8_t)((*mb & (0xF0 >> (4 * (g % 2)))) | (nib << (4 * (g % 2))));
            }
            if (W_out) {
                char* o = (char*)W_out + ((size_t)i * (size_t)ldo + (size_t)(4 * g)) * isz;
                for (int t = 0; t < 4; t++) {
                    if (nib & (1 << t))
                        memcpy(o + t * isz, (const char*)W + (base + (size_t)t) * isz, isz);
                    else
                        memset(o + t * isz, 0, isz);
                }
            }
        }
    }
    return OR_OK;
}

/* Threads the OpenMP loops of this file use (1 without OpenMP): reported beside oracle timings. */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- channel permutation [ORIN7 3.1, 6.3] */

/* Orin NN design, Chapter 7, section 3.1 Step 2 and section 6.3: before the mask is computed, permute
 * the input channels (columns of W, with the matching rows of X) so that large weights share groups of
 * four and 2:4 pruning keeps more of them; the product is unchanged. The pages name no search; this is
 * the one the library defines (a reading, see the design notes):
 *  - the objective of a column order is R = sum over rows m of the retained score in each group: the
 *    sum of its two largest scores (|w|, or the Wanda fl32(|w|) * norm of the column's original
 *    channel), accumulated in double precision row by row in increasing m;
 *  - a sweep is G' - 1 rounds of a round-robin pairing of the G = K/4 groups (G' = G rounded up to
 *    even; position 0 fixed, positions 1..G'-1 rotated by the round; a group paired with the dummy
 *    G'-1 >= G sits out); in each round every pair (A = lower group, B = higher) re-partitions its 8
 *    channels into two groups of four, choosing among the 35 partitions (the channel at A's first slot
 *    stays in A; A's other 3 are a 3-subset of the remaining 7 slots, in lexicographic order, index 0
 *    being the current arrangement) the one with the largest pair objective
 *      S_P = sum_m ( T(A_P, m) + T(B_P, m) ),  T = top-2 sum (fl64(top1 + top2)),
 *    the earliest index on ties (so nothing moves unless it strictly gains); channels keep their slot
 *    order inside A_P and B_P;
 *  - R never decreases.
 * K must be a multiple of 4 (at least 8). perm_out[c] = original column of permuted column c. */
static double top2_sum(const double v[4]) {
    double a = v[0], b = v[1], c = v[2], d = v[3], t;
    /* sort descending (insertion), then the two largest */
    if (b > a) { t = a; a = b; b = t; }
    if (c > b) { t = b; b = c; c = t; if (b > a) { t = a; a = b; b = t; } }
    if (d > c) { t = c; c = d; d = t; if (c > b) { t = b; b = c; c = t; if (b > a) { t = a; a = b; b = t; } } }
    return a + b;
}

static double col_score(const void* W, int dtype, int64_t ldw, int64_t m, int64_t col, int score, const float* norms) {
    double a = fabs(elem_value(W, dtype, (size_t)m * (size_t)ldw + (size_t)col));
    if (score == OR_WANDA) {
        float prod = (float)a * norms[col];
        return (double)prod;
    }
    return a;
}

/* the 35 partitions: 3-subsets of slots {1..7} in lexicographic order */
static void partition_subsets(int subs[35][3]) {
    int n = 0;
    for (int x = 1; x <= 7; x++)
        for (int y = x + 1; y <= 7; y++)
            for (int z = y + 1; z <= 7; z++) { subs[n][0] = x; subs[n][1] = y; subs[n][2] = z; n++; }
}

/* The round-robin schedule: in round r (0 <= r < G' - 1) pair p (0 <= p < G'/2) joins the groups at
 * positions p and G' - 1 - p of the circle in which position 0 is fixed and positions 1 .. G' - 1 hold
 * the groups rotated by r. Returns 1 and the pair (*ga < *gb) when both are real groups, 0 when one is
 * the dummy G' - 1 >= G (that group sits the round out). */
int oracle_perm_pair(int G, int r, int p, int* ga, int* gb) {
    const int Ge = G + (G & 1);
    const int pa = p, pb = Ge - 1 - p;
    int a = pa == 0 ? 0 : 1 + ((pa - 1 + r) % (Ge - 1));
    int b = pb == 0 ? 0 : 1 + ((pb - 1 + r) % (Ge - 1));
    if (a >= G || b >= G) return 0;
    if (a > b) { int t = a; a = b; b = t; }
    *ga = a;
    *gb = b;
    return 1;
}

int oracle_channel_permutation(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                               const float* norms, int sweeps, int32_t* perm_out) {
    if (!W || !perm_out || M < 1 || K < 8 || K % 4 != 0 || ldw < K || sweeps < 0) return OR_EARG;
    if (dtype != OR_BF16 && dtype != OR_FP16 && dtype != OR_FP32 && dtype != OR_I8) return OR_EARG;
    if (score == OR_WANDA && (!norms || dtype == OR_I8)) return OR_EARG;
    if (score != OR_WANDA && score != OR_MAGNITUDE) return OR_EARG;
    const int G = (int)(K / 4), Ge = G + (G & 1);
    int subs[35][3];
    partition_subsets(subs);
    for (int64_t c = 0; c < K; c++) perm_out[c] = (int32_t)c;
    for (int sw = 0; sw < sweeps; sw++) {
        for (int r = 0; r < Ge - 1; r++) {
#pragma omp parallel for schedule(dynamic)
            for (int p = 0; p < Ge / 2; p++) {
                int ga, gb;
                if (!oracle_perm_pair(G, r, p, &ga, &gb)) continue;
                int64_t oc[8];
                for (int i = 0; i < 4; i++) { oc[i] = perm_out[4 * ga + i]; oc[4 + i] = perm_out[4 * gb + i]; }
                double S[35];
                for (int t = 0; t < 35; t++) S[t] = 0.0;
                for (int64_t m = 0; m < M; m++) {
                    double v[8];
                    for (int i = 0; i < 8; i++) v[i] = col_score(W, dtype, ldw, m, oc[i], score, norms);
                    for (int t = 0; t < 35; t++) {
                        double a[4], b[4];
                        int inA[8] = {1, 0, 0, 0, 0, 0, 0, 0}, na = 1, nb = 0;
                        inA[subs[t][0]] = inA[subs[t][1]] = inA[subs[t][2]] = 1;
                        a[0] = v[0];
                        for (int i = 1; i < 8; i++) { if (inA[i]) a[na++] = v[i]; else b[nb++] = v[i]; }
                        S[t] += top2_sum(a) + top2_sum(b);
                    }
                }
                int best = 0;
                for (int t = 1; t < 35; t++) if (S[t] > S[best]) best = t;
                if (best != 0) {
                    int inA[8] = {1, 0, 0, 0, 0, 0, 0, 0}, na = 1, nb = 0;
                    int64_t na_[4], nb_[4];
                    inA[subs[best][0]] = inA[subs[best][1]] = inA[subs[best][2]] = 1;
                    na_[0] = oc[0];
                    for (int i = 1; i < 8; i++) { if (inA[i]) na_[na++] = oc[i]; else nb_[nb++] = oc[i]; }
                    for (int i = 0; i < 4; i++) {
                        perm_out[4 * ga + i] = (int32_t)na_[i];
                        perm_out[4 * gb + i] = (int32_t)nb_[i];
                    }
                }
            }
        }
    }
    return OR_OK;
}

/* Retained objective R of a column order (see above), double precision, rows in increasing order and
 * groups in increasing order within a row. */
double oracle_retained(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score, const float* norms,
                       const int32_t* perm) {
    double R = 0.0;
    for (int64_t m = 0; m < M; m++)
        for (int64_t g = 0; g < K / 4; g++) {
            double v[4];
            for (int i = 0; i < 4; i++) v[i] = col_score(W, dtype, ldw, m, perm ? perm[4 * g + i] : 4 * g + i, score, norms);
            R += top2_sum(v);
        }
    return R;
}

/* ---------------------------------------------------------------- metadata check [ORIN7 6.1] */

/* Every nibble of the M x K region must name two distinct positions in ascending order. Returns
 * the number of bad nibbles (0 when the stream is canonical). val_dtype fixes the layout. */
int64_t oracle_meta_check(const uint8_t* meta, int64_t M, int64_t K, int val_dtype) {
    const int esize = (int)dtype_size(val_dtype);
    int64_t bad = 0;
    for (int64_t i = 0; i < M; i++)
        for (int64_t g = 0; g < K / 4; g++) {
            int nib = get_nibble(meta, i, g, K, esize);
            int i0 = nib & 3, i1 = (nib >> 2) & 3;
            if (!(i0 < i1)) bad++;
        }
    return bad;
}

/* ---------------------------------------------------------------- decompress */

/* Inverse of the compression: the kept value j = 2g + t of row i goes back to column 4g + i_t; the
 * other two columns of the group get +0 (all-zero bits). W_out: M x K row-major, pitch ldw. */
int oracle_decompress(const void* values, const uint8_t* meta, int dtype, int64_t M, int64_t K, void* W_out,
                      int64_t ldw) {
    if (!values || !meta || !W_out || M < 0 || K < 0 || K % 16 != 0 || ldw < K) return OR_EARG;
    const size_t sz = dtype_size(dtype);
    if (sz == 0 || dtype == OR_I32) return OR_EARG;
    if (oracle_meta_check(meta, M, K, dtype) != 0) return OR_EMETA;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; i++) {
        char* orow = (char*)W_out + (size_t)i * (size_t)ldw * sz;
        memset(orow, 0, (size_t)K * sz);
        for (int64_t g = 0; g < K / 4; g++) {
            int nib = get_nibble(meta, i, g, K, (int)sz);
            int pos[2] = {nib & 3, (nib >> 2) & 3};
            for (int t = 0; t < 2; t++) {
                const char* src = (const char*)values + values_offset(i, (2 * g + t) * (int64_t)sz, K, (int)sz);
                memcpy(orow + (size_t)(4 * g + pos[t]) * sz, src, sz);
            }
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------- sparse x dense GEMM */

/* Exact value of kept value j of row i. */
static double kept_value(const void* values, int dtype, int64_t i, int64_t j, int64_t K) {
    const int sz = (int)dtype_size(dtype);
    const char* p = (const char*)values + values_offset(i, j * sz, K, sz);
    switch (dtype) {
    case OR_BF16: { uint16_t h; memcpy(&h, p, 2); return bf16_value(h); }
    case OR_I8: return (double)*(const int8_t*)p;
    }
    return NAN;
}

/* Dense row i of the pruned weight, as exact doubles (zeros at pruned slots). */
static void dense_row(const void* values, const uint8_t* meta, int dtype, int64_t i, int64_t K, double* w) {
    for (int64_t k = 0; k < K; k++) w[k] = 0.0;
    for (int64_t g = 0; g < K / 4; g++) {
        int nib = get_nibble(meta, i, g, K, (int)dtype_size(dtype));
        w[4 * g + (nib & 3)] = kept_value(values, dtype, i, 2 * g, K);
        w[4 * g + ((nib >> 2) & 3)] = kept_value(values, dtype, i, 2 * g + 1, K);
    }
}

/* Y = W_2:4 . X for a list of output rows, in double [ORIN7 2.1 Step 3; NVBLOG Figure 1].
 * values: bf16, meta: as above; X: bf16 K x N row-major (pitch ldx).
 * rows[r] (r < nrows) names the output row; Y is nrows x N (row pitch N), double.
 * The row is rebuilt densely and each Y[r, n] sums W[m, k] * X[k, n] over k in ascending order;
 * every product of two bf16 numbers is exact in double. */
int oracle_gemm_bf16(const uint16_t* values, const uint8_t* meta, int64_t M, int64_t K, const uint16_t* X,
                     int64_t N, int64_t ldx, const int64_t* rows, int64_t nrows, double* Y) {
    if (!values || !meta || !X || !rows || !Y || M < 0 || K < 0 || K % 16 != 0 || N < 0 || ldx < N) return OR_EARG;
    for (int64_t r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= M) return OR_EARG;
    if (oracle_meta_check(meta, M, K, OR_BF16) != 0) return OR_EMETA;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; r++) {
            dense_row(values, meta, OR_BF16, rows[r], K, w);
            double* y = Y + (size_t)r * (size_t)N;
            for (int64_t n = 0; n < N; n++) y[n] = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const uint16_t* xr = X + (size_t)k * (size_t)ldx;
                for (int64_t n = 0; n < N; n++) y[n] += w[k] * bf16_value(xr[n]);
            }
        }
        free(w);
    }
    return OR_OK;
}

/* int8 sparse GEMM with int32 accumulation and per-output-channel dequant [FORUM; ORIN7 3.1 Step 4].
 * acc[r, n] = sum_k W[m, k] * X[k, n] exactly (int64; it must fit int32, else OR_EOVERFLOW).
 * If Y is not NULL, Y[r, n] = fl32( fl32(acc) * scale[m] ), one single-precision multiply. */
int oracle_gemm_i8(const int8_t* values, const uint8_t* meta, int64_t M, int64_t K, const int8_t* X, int64_t N,
                   int64_t ldx, const float* scale, const int64_t* rows, int64_t nrows, int64_t* acc_out, float* Y) {
    if (!values || !meta || !X || !rows || !acc_out || M < 0 || K < 0 || K % 16 != 0 || N < 0 || ldx < N)
        return OR_EARG;
    if (Y && !scale) return OR_EARG;
    for (int64_t r = 0; r < nrows; r++)
        if (rows[r] < 0 || rows[r] >= M) return OR_EARG;
    if (oracle_meta_check(meta, M, K, OR_I8) != 0) return OR_EMETA;
    int overflow = 0;
#pragma omp parallel reduction(| : overflow)
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; r++) {
            dense_row(values, meta, OR_I8, rows[r], K, w);
            int64_t* a = acc_out + (size_t)r * (size_t)N;
            for (int64_t n = 0; n < N; n++) a[n] = 0;
            for (int64_t k = 0; k < K; k++) {
                int64_t wk = (int64_t)w[k];
                const int8_t* xr = X + (size_t)k * (size_t)ldx;
                for (int64_t n = 0; n < N; n++) a[n] += wk * (int64_t)xr[n];
            }
            for (int64_t n = 0; n < N; n++) {
                if (a[n] > INT32_MAX || a[n] < INT32_MIN) overflow = 1;
                if (Y) {
                    float accf = (float)(int32_t)a[n];
                    float prod = accf * scale[rows[r]];
                    Y[(size_t)r * (size_t)N + (size_t)n] = prod;
                }
            }
        }
        free(w);
    }
    return overflow ? OR_EOVERFLOW : OR_OK;
}

/* Exposed for the tests that pin the format conversions against independent references. */
uint16_t oracle_fp32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return fp32_to_bf16_rne(u);
}
double oracle_fp16_value(uint16_t h) { return fp16_value(h); }
