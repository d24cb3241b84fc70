"""GPU parity of the dense reference GEMM that bench.py times beside the sparse one (include/sp24_bench.h):
the dense tiled copy equals an independent numpy statement of its layout bit for bit, and the dense GEMM of
the pruned weight equals the oracle's fp64 product of the same bf16 inputs within the fp32 summation bound
(element by element) and 1e-3 Frobenius; bf16 output equals the kernel's own fp32 result rounded to nearest
even."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import bf16_to_f64, dev, fp32_sum_bound, frob_rel, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def dense_tiled_ref(Wd, M, K):
    """numpy statement of the tiled order: tile (row block b, 32-column tile t) at (b * K/32 + t) KB; byte
    16 l + 2 e of a tile holds row 16 b + l % 16, column 32 t + 8 (l // 16) + e; rows past M are zero."""
    Mp = (M + 15) // 16 * 16
    P = np.zeros((Mp, K), np.uint16)
    P[:M] = Wd
    # (b, r, t, q, e) -> (b, t, q, r, e)
    return P.reshape(Mp // 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)


@pytest.mark.parametrize("M,K,N,ldx", [(300, 256, 130, 256), (257, 512, 513, 520), (1000, 640, 777, 640),
                                       (96, 64, 70, 72), (8192, 512, 4096, 512)])
def test_dense_reference(M, K, N, ldx):
    rng = np.random.default_rng(M + K + N)
    W = synth.normal_bf16(int(rng.integers(1 << 30)), (M, K), 0.02)
    X = synth.normal_bf16(int(rng.integers(1 << 30)), (N, K))
    rv, rm = oracle.prune_compress(W, oracle.BF16)
    Wd = oracle.decompress(rv, rm, oracle.BF16, M, K)
    say(f"dense reference M={M} K={K} N={N} ldx={ldx}")
    Wt = sp.sp24_bench_dense_tile(dev(Wd, "bf16"))
    assert np.array_equal(host_bits(Wt), dense_tiled_ref(Wd, M, K))
    Xp = np.zeros((N, ldx), np.uint16)
    Xp[:, :K] = X
    Xd = dev(Xp, "bf16")[:, :K]
    Yf = sp.sp24_bench_gemm_dense_bf16(Wt, M, Xd, out_dtype=torch.float32)
    Yb = sp.sp24_bench_gemm_dense_bf16(Wt, M, Xd, out_dtype=torch.bfloat16)
    rows = np.arange(M) if M * K * N <= 2e9 else np.unique(np.concatenate([np.arange(0, M, 97), [M - 1]]))
    Y64 = oracle.gemm_bf16(rv, rm, X, M, rows=rows, layout="token")  # N x len(rows)
    r = torch.from_numpy(rows).cuda()
    yf = host_bits(Yf[:, r])
    bound = fp32_sum_bound(np.abs(bf16_to_f64(X)) @ np.abs(bf16_to_f64(Wd[rows])).T, K)
    assert np.all(np.abs(yf.astype(np.float64) - Y64) <= bound)
    assert frob_rel(yf, Y64) <= 1e-3
    assert np.array_equal(host_bits(Yb), synth.f32_to_bf16_bits(host_bits(Yf)))


@pytest.mark.parametrize("nbytes", [16, 4096, 1000000 * 16 + 48, 19 * (1 << 20)])
def test_stream_read_reads_every_word(nbytes):
    # the floor kernel bench.py times: the XOR of its per-workgroup words is the XOR of every 16-byte word
    rng = np.random.default_rng(nbytes % 1000)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    say(f"stream read {nbytes} bytes")
    src = dev(words.view(np.int32))
    sink = host_bits(sp.sp24_bench_stream_read(src)).view(np.uint32).reshape(-1, 4)
    x = np.bitwise_xor.reduce(sink, axis=0)
    want = np.bitwise_xor.reduce(words.reshape(-1, 4), axis=0)
    assert np.array_equal(x, want)
