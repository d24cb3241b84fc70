"""GPU parity at the degenerate sizes: a single output channel (M = 1, fifteen padded rows in the compressed
row block), the smallest K (16: one group column of a quarter tile), and one token, through every GEMM kernel of
both dtypes in both layouts: the direct, few-token, skinny and tiled kernels (the kernel is chosen from the
shape). Whole outputs against the oracle: int8 bit-exact, bf16 within the fp32 summation bound of the fp64
product and equal to the same kernel's fp32 result rounded to nearest even, the fused int8 epilogue without
GELU bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import bf16_to_f64, dev, fp32_sum_bound, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# M, K, N, layout
BF16_SHAPES = [
    (1, 16, 1, "feature"), (1, 16, 1, "token"),        # the smallest product (direct / few-token kernels)
    (1, 64, 16, "token"), (1, 64, 2, "token"),         # few-token kernels
    (1, 128, 40, "feature"), (1, 128, 40, "token"),    # skinny kernels
    (1, 64, 72, "feature"), (1, 64, 100, "token"),     # tiled kernels, one row of one tile
    (17, 16, 70, "feature"), (17, 64, 70, "token"),    # one row past a block (direct; tiled)
    (1, 8192, 129, "token"),                           # one row over a long K
]


@pytest.mark.parametrize("M,K,N,layout", BF16_SHAPES)
def test_bf16_degenerate(M, K, N, layout):
    W = synth.normal_bf16(M * 7 + K + N, (M, K), 0.02)
    X = synth.normal_bf16(M + K + N, (K, N))
    v, m = oracle.prune_compress(W, oracle.BF16)
    say(f"degenerate bf16 M={M} K={K} N={N} {layout}")
    vd, md = sp.sp24_prune_compress(dev(W, "bf16"))
    assert np.array_equal(host_bits(vd), v) and np.array_equal(host_bits(md), m)
    Xd = dev(X if layout == "feature" else np.ascontiguousarray(X.T), "bf16")
    Yf = host_bits(sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout=layout, out_dtype=torch.float32))
    Yb = host_bits(sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout=layout, out_dtype=torch.bfloat16))
    if layout == "token":
        Yf, Yb = Yf.T, Yb.T
    Y64 = oracle.gemm_bf16(v, m, X, M)
    dense = bf16_to_f64(oracle.decompress(v, m, oracle.BF16, M, K))
    bound = fp32_sum_bound(np.abs(dense) @ np.abs(bf16_to_f64(X)), K)
    assert np.all(np.abs(Yf.astype(np.float64) - Y64) <= bound)
    assert np.array_equal(Yb, synth.f32_to_bf16_bits(np.ascontiguousarray(Yf)))


# M, K, N, layout
I8_SHAPES = [
    (1, 16, 1, "feature"), (1, 16, 3, "token"),        # direct kernel (K below one 128-column tile)
    (1, 128, 1, "token"), (1, 128, 16, "token"), (1, 256, 64, "token"),  # few-token kernel
    (1, 128, 80, "feature"), (1, 128, 70, "token"),    # tiled kernels
    (17, 128, 100, "token"), (1, 8192, 144, "feature"), (3, 384, 67, "feature"),  # the last: direct
]


@pytest.mark.parametrize("M,K,N,layout", I8_SHAPES)
def test_int8_degenerate(M, K, N, layout):
    rng = np.random.default_rng(M * 13 + K + N)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(K, N), dtype=np.int8)
    scale = (rng.random(M) * 1e-3 + 1e-5).astype(np.float32)
    bias = (rng.standard_normal(M) * 0.02).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    say(f"degenerate int8 M={M} K={K} N={N} {layout}")
    vd, md = sp.sp24_prune_compress(dev(W))
    assert np.array_equal(host_bits(vd), v) and np.array_equal(host_bits(md), m)
    Xh = X if layout == "feature" else np.ascontiguousarray(X.T)
    Xd = dev(Xh)
    acc, Y = oracle.gemm_i8(v, m, Xh, M, scale, layout=layout)
    got_acc = host_bits(sp.sp24_gemm_i8_ex(vd, md, M, Xd, layout=layout))
    got_y = host_bits(sp.sp24_gemm_i8_ex(vd, md, M, Xd, scale=dev(scale), layout=layout))
    assert np.array_equal(got_acc.astype(np.int64), acc)
    assert np.array_equal(got_y.view(np.uint32), np.ascontiguousarray(Y).view(np.uint32))
    # the fused epilogue with bias and requantized int8 output (no GELU: every step one IEEE rounding)
    ref = oracle.gemm_i8_fused(v, m, Xh, M, scale, bias, gelu=False, out_scale=0.05, layout=layout)
    got_q = host_bits(sp.sp24_gemm_i8_fused(vd, md, M, Xd, dev(scale), bias=dev(bias), out_dtype=torch.int8,
                                            out_scale=0.05, layout=layout))
    assert np.array_equal(got_q, ref["q"])
