"""GPU parity of the int8 GEMM's fused FFN epilogue (sp24_gemm_i8_fused): dequant, optional bias,
optional GELU, and fp32 / bf16 / int8 output, in both layouts and through the tiled and direct kernels.

Bars: without GELU every step is a single IEEE rounding on both sides, so fp32 output and int8 codes
are bit-exact and bf16 output is the nearest-even rounding of the oracle's fp32 value. With GELU the
kernel uses the Abramowitz & Stegun 7.1.26 approximation (expanded in 1 - t): fp32 output within 8 * 2^-24 * |y| (+1e-30) of the float64 GELU of the same
fp32 input; bf16 output equal to the nearest-even rounding of the same kernel's fp32 output; int8 codes
within 1 of the reference everywhere and equal wherever the reference y / out_scale is farther than the
error bound from a rounding boundary."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import dev, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu

GELU_REL = 8 * 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


SHAPES = [
    # M, K, N, layout: tiled (N > 64, K % 128 == 0 for token-major), direct (small N, K tails), ragged
    (257, 512, 513, "feature"),
    (300, 640, 200, "token"),
    (96, 256, 130, "feature"),
    (33, 48, 17, "token"),
    (40, 208, 90, "feature"),
    (200, 256, 12, "token"),   # few-token kernel: one fragment
    (150, 384, 40, "token"),   # few-token kernel: three fragments
    (520, 1152, 1000, "token"),
    (16400, 256, 20, "token"),  # few-token kernel, two row blocks per workgroup, odd block count (1025)
    (8200, 256, 10, "token"),   # few-token LDS ring, four-wave workgroups (513 row blocks)
    (16400, 128, 2, "token"),   # few-token LDS ring for one or two tokens (1025 row blocks)
    (2300, 256, 8200, "token"),  # 128-wide tiles, two workgroups per compute unit (585 tiles, ragged)
    (11008, 256, 12, "token"),  # few-token LDS ring, units of three row blocks
]


def _inputs(M, K, N, layout, seed):
    rng = np.random.default_rng(seed)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(N, K) if layout == "token" else (K, N), dtype=np.int8)
    scale = (rng.random(M) * 2e-4 + 1e-5).astype(np.float32)
    bias = rng.standard_normal(M).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    return X, scale, bias, v, m


@pytest.mark.parametrize("M,K,N,layout", SHAPES)
@pytest.mark.parametrize("use_bias", [False, True])
def test_fused_no_gelu_bit_exact(M, K, N, layout, use_bias):
    X, scale, bias, v, m = _inputs(M, K, N, layout, M + K + N)
    b = bias if use_bias else None
    out_scale = 0.05
    ref = oracle.gemm_i8_fused(v, m, X, M, scale, b, out_scale=out_scale, layout=layout)
    say(f"gemm_i8_fused M={M} K={K} N={N} {layout} bias={use_bias}")
    args = (dev(v), dev(m), M, dev(X), dev(scale))
    kw = dict(bias=dev(b) if use_bias else None, layout=layout)
    y32 = host_bits(sp.sp24_gemm_i8_fused(*args, out_dtype=torch.float32, **kw))
    y16 = host_bits(sp.sp24_gemm_i8_fused(*args, out_dtype=torch.bfloat16, **kw))
    q = host_bits(sp.sp24_gemm_i8_fused(*args, out_dtype=torch.int8, out_scale=out_scale, **kw))
    assert np.array_equal(y32.view(np.uint32), ref["y32"].view(np.uint32))
    assert np.array_equal(y16, synth.f32_to_bf16_bits(ref["y32"]))
    assert np.array_equal(q, ref["q"])


@pytest.mark.parametrize("M,K,N,layout", SHAPES)
def test_fused_gelu(M, K, N, layout):
    X, scale, bias, v, m = _inputs(M, K, N, layout, 3 * M + K + N)
    # the next layer's input scale: 99.9 % of the activations inside the int8 range
    y_ref = oracle.gemm_i8_fused(v, m, X, M, scale, bias, gelu=True, layout=layout)["y"]
    out_scale = float(np.float32(np.quantile(np.abs(y_ref), 0.999) / 127))
    ref = oracle.gemm_i8_fused(v, m, X, M, scale, bias, gelu=True, out_scale=out_scale, layout=layout)
    say(f"gemm_i8_fused GELU M={M} K={K} N={N} {layout}")
    args = (dev(v), dev(m), M, dev(X), dev(scale))
    kw = dict(bias=dev(bias), activation="gelu", layout=layout)
    y32 = host_bits(sp.sp24_gemm_i8_fused(*args, out_dtype=torch.float32, **kw))
    y16 = host_bits(sp.sp24_gemm_i8_fused(*args, out_dtype=torch.bfloat16, **kw))
    q = host_bits(sp.sp24_gemm_i8_fused(*args, out_dtype=torch.int8, out_scale=out_scale, **kw)).astype(np.int32)
    bound = GELU_REL * np.abs(ref["y32"].astype(np.float64)) + 1e-30
    err = np.abs(y32.astype(np.float64) - ref["y"])
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound)}"
    assert np.array_equal(y16, synth.f32_to_bf16_bits(y32))
    qr = ref["q"].astype(np.int32)
    assert np.all(np.abs(q - qr) <= 1)
    d = ref["y"] / np.float64(np.float32(out_scale))
    far = np.abs(d - np.floor(d) - 0.5) > bound / np.float32(out_scale) + 1e-6
    far &= np.abs(d) < 126.5  # away from the clamp
    assert np.array_equal(q[far], qr[far])
    assert far.mean() > 0.98


def test_fused_batched_token_major_int8_chain():
    # the FFN chain: W1's fused output (bias + GELU, int8 codes at the next layer's scale) feeds W2
    rng = np.random.default_rng(77)
    B, M1, K1, N = 2, 256, 128, 96
    W1 = rng.integers(-128, 128, size=(M1, K1), dtype=np.int8)
    W2 = rng.integers(-128, 128, size=(64, M1), dtype=np.int8)
    X = rng.integers(-128, 128, size=(B, N, K1), dtype=np.int8)
    s1 = (rng.random(M1) * 1e-4).astype(np.float32)
    b1 = rng.standard_normal(M1).astype(np.float32)
    s2 = (rng.random(64) * 1e-3).astype(np.float32)
    v1, m1 = oracle.prune_compress(W1, oracle.I8)
    v2, m2 = oracle.prune_compress(W2, oracle.I8)
    say("gemm_i8_fused batched token-major chain")
    H = sp.sp24_gemm_i8_fused(dev(v1), dev(m1), M1, dev(X), dev(s1), bias=dev(b1), activation="gelu",
                              out_dtype=torch.int8, out_scale=0.05, layout="token")
    Y = host_bits(sp.sp24_gemm_i8_fused(dev(v2), dev(m2), 64, H, dev(s2), layout="token"))
    h = host_bits(H)
    for b in range(B):
        ref_h = oracle.gemm_i8_fused(v1, m1, X[b], M1, s1, b1, gelu=True, out_scale=0.05, layout="token")["q"]
        assert np.all(np.abs(h[b].astype(np.int32) - ref_h.astype(np.int32)) <= 1)
        # the second layer is bit-exact on the codes the GPU produced
        ref_y = oracle.gemm_i8_fused(v2, m2, h[b], 64, s2, layout="token")["y"]
        assert np.array_equal(Y[b].view(np.uint32), ref_y.view(np.uint32))


@pytest.mark.parametrize("N", [1, 40])
def test_fused_batched_two_blocks_per_workgroup(N):
    # the few-token kernel's R = 2 launch (1025 row blocks) over a batch of 3 token-major inputs, with bias,
    # GELU and int8 output
    rng = np.random.default_rng(90 + N)
    B, M, K = 3, 16400, 256
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(B, N, K), dtype=np.int8)
    scale = (rng.random(M) * 2e-4 + 1e-5).astype(np.float32)
    bias = rng.standard_normal(M).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    out_scale = 0.02
    say(f"gemm_i8_fused batched R=2 M={M} K={K} N={N} B={B}")
    q = host_bits(sp.sp24_gemm_i8_fused(dev(v), dev(m), M, dev(X), dev(scale), bias=dev(bias), activation="gelu",
                                        out_dtype=torch.int8, out_scale=out_scale, layout="token")).astype(np.int32)
    y = host_bits(sp.sp24_gemm_i8_fused(dev(v), dev(m), M, dev(X), dev(scale), bias=dev(bias), layout="token"))
    for b in range(B):
        ref = oracle.gemm_i8_fused(v, m, X[b], M, scale, bias, gelu=True, out_scale=out_scale, layout="token")
        assert np.all(np.abs(q[b] - ref["q"].astype(np.int32)) <= 1)
        assert np.mean(q[b] == ref["q"]) > 0.98
        ref_nb = oracle.gemm_i8_fused(v, m, X[b], M, scale, bias, layout="token")["y32"]
        assert np.array_equal(y[b].view(np.uint32), ref_nb.view(np.uint32))
