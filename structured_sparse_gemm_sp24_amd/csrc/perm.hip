// Input-channel permutation before pruning (Orin NN design, Chapter 7, section 3.1 Step 2 "Channel
// Permutation" and section 6.3): find an order of W's columns (input channels) in which 2:4 pruning
// keeps more of the weights' score; the product is unchanged when X's rows (or the previous layer's
// output channels) follow the same order.
//
// The search, as the library defines it (the pages name none): the objective of a column order is the
// sum over rows m of the two largest scores of every group of four, accumulated in double precision
// row by row. A sweep is G' - 1 rounds of a round-robin pairing of the G = K/4 groups (G' = G rounded
// up to even; position 0 fixed, positions 1..G'-1 rotated by the round, a group paired with the dummy
// sits out). In a round, each pair (A = lower group, B = higher) re-partitions its 8 channels among the
// 35 splits into two groups of four (A's first slot stays in A; A's other three are a 3-subset of the
// remaining 7 slots in lexicographic order; index 0 is the current split) and takes the split of
// largest pair objective, the lowest index on ties, so nothing moves unless the objective strictly
// grows. The pairs of a round are disjoint, so a round is one launch with one workgroup per pair: the
// per-row pair objectives of all 35 splits are computed in parallel into LDS, then lane t of wave 0
// adds split t's column row by row, in row order -- the defined double-precision sum, so the decisions
// are the defined ones -- and thread 0 rewrites the pair's 8 entries of perm. Everything stays on the
// stream; nothing is read back.
#include "sp24_device.h"
#include "sp24_launch.h"

namespace sp24 {
namespace perm_search {

constexpr int RB = 128;      // rows per LDS block
constexpr int NSPLIT = 35;  // splits of 8 channels into two groups of four, slot 0 in A

// Score of element (m, col) as an fp32 value: |w| (exact for every dtype), or fl32(|w|) * norm[col] for
// Wanda. The top-2 choice is exact in fp32; the sums are taken in double.
template <int DT, bool WANDA>
__device__ __forceinline__ float score(const void* W, int64_t ldw, int64_t m, int64_t col, const float* norms) {
    const int64_t i = m * ldw + col;
    float a;
    if constexpr (DT == 2) {
        a = fabsf(reinterpret_cast<const float*>(W)[i]);
    } else if constexpr (DT == 3) {
        const int v = reinterpret_cast<const int8_t*>(W)[i];
        return (float)(v < 0 ? -v : v);
    } else if constexpr (DT == 1) {
        a = f16_to_f32(reinterpret_cast<const uint16_t*>(W)[i] & 0x7FFFu);
    } else {
        a = bf16_to_f32(reinterpret_cast<const uint16_t*>(W)[i] & 0x7FFFu);
    }
    if constexpr (WANDA) {
#pragma clang fp contract(off)
        return __fmul_rn(a, norms[col]);
    }
    return a;
}

// Split n's A group: slot 0 plus the n-th 3-subset {x < y < z} of slots 1..7 in lexicographic order
// (i = 0, 1, 2 gives x, y, z); B is the complement (i = 0..3, ascending).
constexpr int split_a(int n, int i) {
    int c = 0;
    for (int x = 1; x <= 7; x++)
        for (int y = x + 1; y <= 7; y++)
            for (int z = y + 1; z <= 7; z++) {
                if (c == n) return i == 0 ? x : i == 1 ? y : z;
                c++;
            }
    return -1;
}
constexpr int split_b(int n, int i) {
    int c = 0;
    for (int s = 1; s < 8; s++)
        if (s != split_a(n, 0) && s != split_a(n, 1) && s != split_a(n, 2)) {
            if (c == i) return s;
            c++;
        }
    return -1;
}

// fl64(top1 + top2) of four fp32 scores (max/min select exactly; two fp32 values convert exactly).
__device__ __forceinline__ double top2_sum(float v0, float v1, float v2, float v3) {
    const float a = fmaxf(v0, v1), b = fminf(v0, v1), c = fmaxf(v2, v3), d = fminf(v2, v3);
    const float t1 = fmaxf(a, c), t2 = fmaxf(fminf(a, c), fmaxf(b, d));
    return (double)t1 + (double)t2;
}

// One row's pair objective T(A_n) + T(B_n) for splits N..E-1, written to out[N..E-1].
template <int N, int E>
__device__ __forceinline__ void row_objectives(const float (&v)[8], double* out) {
    if constexpr (N < E) {
        constexpr int x = split_a(N, 0), y = split_a(N, 1), z = split_a(N, 2);
        constexpr int p = split_b(N, 0), q = split_b(N, 1), r = split_b(N, 2), u = split_b(N, 3);
        out[N] = top2_sum(v[0], v[x], v[y], v[z]) + top2_sum(v[p], v[q], v[r], v[u]);
        row_objectives<N + 1, E>(v, out);
    }
}

__global__ void init_kernel(int32_t* perm, int64_t K) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c < K) perm[c] = (int32_t)c;
}

// One round: workgroup p handles the p-th pair of the round. Per block of RB rows, the 256 threads
// compute every row's 35 pair objectives into LDS (threads 0..127 splits 0..17, threads 128..255 splits
// 18..34, one row each); then lanes 0..34 of wave 0 add their split's column to a running double sum
// row by row, in row order.
template <int DT, bool WANDA>
__global__ __launch_bounds__(256) void round_kernel(const void* __restrict__ W, int64_t ldw, int64_t M, int G, int round,
                                                    const float* __restrict__ norms, int32_t* __restrict__ perm) {
    __shared__ double c[RB][NSPLIT];
    __shared__ double S[NSPLIT];
    const int Ge = G + (G & 1);
    const int qa = blockIdx.x, qb = Ge - 1 - blockIdx.x;
    int ga = qa == 0 ? 0 : 1 + ((qa - 1 + round) % (Ge - 1));
    int gb = qb == 0 ? 0 : 1 + ((qb - 1 + round) % (Ge - 1));
    if (ga >= G || gb >= G) return;  // whole workgroup: paired with the dummy group
    if (ga > gb) {
        const int t = ga;
        ga = gb;
        gb = t;
    }
    int64_t oc[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        oc[i] = perm[4 * ga + i];
        oc[4 + i] = perm[4 * gb + i];
    }
    const int t = threadIdx.x;
    const int lr = t & (RB - 1);
    double s = 0.0;
    for (int64_t m0 = 0; m0 < M; m0 += RB) {
        const int rows = (int)(M - m0 < RB ? M - m0 : RB);
        if (lr < rows) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) v[i] = score<DT, WANDA>(W, ldw, m0 + lr, oc[i], norms);
            if (t < RB) row_objectives<0, 18>(v, c[lr]);
            else row_objectives<18, NSPLIT>(v, c[lr]);
        }
        __syncthreads();
        if (t < NSPLIT) {
#pragma unroll 8
            for (int r = 0; r < rows; r++) s += c[r][t];
        }
        __syncthreads();
    }
    if (t < NSPLIT) S[t] = s;
    __syncthreads();
    if (t == 0) {
        int best = 0;
        for (int u = 1; u < NSPLIT; u++)
            if (S[u] > S[best]) best = u;
        if (best != 0) {
            int mask = 1, n = 0;
            for (int x = 1; x <= 7; x++)
                for (int y = x + 1; y <= 7; y++)
                    for (int z = y + 1; z <= 7; z++) {
                        if (n == best) mask = 1 | (1 << x) | (1 << y) | (1 << z);
                        n++;
                    }
            int na = 0, nb = 0;
            for (int i = 0; i < 8; i++) {
                if ((mask >> i) & 1) perm[4 * ga + na++] = (int32_t)oc[i];
                else perm[4 * gb + nb++] = (int32_t)oc[i];
            }
        }
    }
}

template <int DT, bool WANDA>
hipError_t run(const void* W, int64_t M, int64_t K, int64_t ldw, const float* norms, int sweeps, int32_t* perm,
               hipStream_t s) {
    hipLaunchKernelGGL(init_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, perm, K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = (int)(K / 4), Ge = G + (G & 1);
    for (int sw = 0; sw < sweeps; sw++)
        for (int r = 0; r < Ge - 1; r++) {
            hipLaunchKernelGGL((round_kernel<DT, WANDA>), dim3((unsigned)(Ge / 2)), dim3(256), 0, s, W, ldw, M, G, r, norms,
                               perm);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    return hipSuccess;
}

}  // namespace perm_search

hipError_t launch_channel_permutation(const void* W, int dtype, int64_t M, int64_t K, int64_t ldw, int score,
                                      const float* norms, int sweeps, int32_t* perm, hipStream_t s) {
    const bool wanda = score == 1;
    switch (dtype) {
    case 0: return wanda ? perm_search::run<0, true>(W, M, K, ldw, norms, sweeps, perm, s)
                         : perm_search::run<0, false>(W, M, K, ldw, norms, sweeps, perm, s);
    case 1: return wanda ? perm_search::run<1, true>(W, M, K, ldw, norms, sweeps, perm, s)
                         : perm_search::run<1, false>(W, M, K, ldw, norms, sweeps, perm, s);
    case 2: return wanda ? perm_search::run<2, true>(W, M, K, ldw, norms, sweeps, perm, s)
                         : perm_search::run<2, false>(W, M, K, ldw, norms, sweeps, perm, s);
    case 3: return perm_search::run<3, false>(W, M, K, ldw, norms, sweeps, perm, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace sp24
