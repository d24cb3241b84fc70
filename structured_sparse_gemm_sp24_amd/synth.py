"""Seeded synthetic inputs for the 2:4 sparse path (shared by tests, smoke check and benchmark).

This module only draws numbers and prepares caller-side inputs. It holds none of the path's own
arithmetic (no scoring, selection, compression or contraction), imports neither the oracle nor the
HIP binding, and gives both sides the same bytes.

Draws use numpy's PCG64 ``default_rng(seed)`` in row-major order, in float32, then round to bf16
(round to nearest even, done by torch's CPU conversion).

Workload shapes stand in for the layers the pages name as the ones worth sparsifying: Transformer
projections and FFN Linear layers of ViT-B/16 and BERT-base, and large LLM projections (Orin NN
design book, Chapter 7, section 2.2 A; CSDN Q&A on "4:2" sparsity, section 3). No dataset,
checkpoint or calibration corpus is used.

The int8 preparation (per-output-channel and per-tensor symmetric scales covering 99.99 % of the
magnitudes, per the quantization section of the NVIDIA technical blog on Ampere structured sparsity)
is also a caller-side step: the sparse int8 GEMM takes already quantized operands plus one fp32
scale per output channel.
"""
from __future__ import annotations

import numpy as np
import torch

# ------------------------------------------------------------------ format helpers


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest even) with torch's CPU conversion; returns uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def normal_bf16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, shape, sigma))


def heavy_tailed_bf16(seed: int, K: int, N: int) -> np.ndarray:
    """X[j, n] = c_j * t_jn with c_j ~ LogNormal(0, 1) per input channel and t ~ Student-t(3) i.i.d.,
    giving heavy-tailed per-channel norms (the regime where Wanda's activation term matters)."""
    rng = np.random.default_rng(seed)
    c = rng.lognormal(mean=0.0, sigma=1.0, size=(K, 1)).astype(np.float32)
    t = rng.standard_t(3, size=(K, N)).astype(np.float32)
    return f32_to_bf16_bits(c * t)


# ------------------------------------------------------------------ int8 preparation (caller side)

QMAX = 127


def symmetric_scale(absvals: np.ndarray, coverage: float = 0.9999) -> float:
    """Scale s so that `coverage` of the magnitudes fit in [-127 s, 127 s] (numpy's linear-interpolation
    quantile). Returned as a float32 value."""
    q = float(np.quantile(np.abs(absvals).astype(np.float64), coverage))
    if q == 0.0:
        q = 1.0
    return float(np.float32(q / QMAX))


def quantize_sym(x: np.ndarray, s) -> np.ndarray:
    """q = clamp(round_half_even(x / s), -127, 127), the division in float64."""
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    q = np.rint(np.asarray(x, dtype=np.float64) / s64)
    return np.clip(q, -QMAX, QMAX).astype(np.int8)


def quantize_rows(W: np.ndarray, coverage: float = 0.9999):
    """Per-output-channel (row) symmetric int8: returns (q int8 M x K, s float32[M])."""
    W = np.asarray(W, dtype=np.float32)
    s = np.array([symmetric_scale(W[m], coverage) for m in range(W.shape[0])], dtype=np.float32)
    return quantize_sym(W, s[:, None]), s


def quantize_tensor(X: np.ndarray, coverage: float = 0.9999):
    """Per-tensor symmetric int8: returns (q int8, s float32)."""
    s = symmetric_scale(np.asarray(X, dtype=np.float32).ravel(), coverage)
    return quantize_sym(X, s), np.float32(s)


def dequant_scales(s_w: np.ndarray, s_x) -> np.ndarray:
    """scale[m] = fl32(s_w[m] * s_x), the product taken in float64 and rounded once."""
    return (np.asarray(s_w, np.float32).astype(np.float64) * float(np.float32(s_x))).astype(np.float32)


# ------------------------------------------------------------------ the workloads

WORKLOADS = {
    "single_linear_256": dict(M=256, K=256, N=64),
    "vit_b16_fc1": dict(M=3072, K=768, N=6304),
    "bert_ffn_int8_w1": dict(M=3072, K=768, N=8192),
    "bert_ffn_int8_w2": dict(M=768, K=3072, N=8192),
    "llm_proj_11008x4096": dict(M=11008, K=4096, Ncal=2048, N=(1, 16, 4096)),
    "llm_proj_4096x4096": dict(M=4096, K=4096, Ncal=2048, N=(1, 16, 4096)),
    "ffn_28672x8192": dict(M=28672, K=8192, N=(8, 64, 512, 8192)),
}


def single_linear_256():
    """W 256x256 fp32 ~N(0,1) (seed 1); X 256x64 fp32 ~N(0,1) (seed 2), also as bf16."""
    W = normal_f32(1, (256, 256))
    Xf = normal_f32(2, (256, 64))
    return dict(W_f32=W, X_f32=Xf, X_bf16=f32_to_bf16_bits(Xf))


def vit_b16_fc1():
    """ViT-B/16 MLP fc1: W 3072x768 bf16 ~N(0, 0.02^2) (seed 11); X 768x6304 bf16 ~N(0,1) (seed 12),
    N = 32 images x 197 tokens."""
    return dict(W_bf16=normal_bf16(11, (3072, 768), 0.02), X_bf16=normal_bf16(12, (768, 6304)))


def bert_ffn_int8_dense():
    """BERT-base FFN pair before pruning/quantization: W1 3072x768 (seed 21), W2 768x3072 (seed 22)
    fp32 ~N(0, 0.02^2); X1 768x8192 (seed 23), X2 3072x8192 (seed 24) fp32 ~N(0,1), N = 64 x 128.
    X2 is an independent draw (the two GEMMs are benchmarked independently)."""
    return dict(W1_f32=normal_f32(21, (3072, 768), 0.02), W2_f32=normal_f32(22, (768, 3072), 0.02),
                X1_f32=normal_f32(23, (768, 8192)), X2_f32=normal_f32(24, (3072, 8192)))


def llm_proj_int8_dense():
    """LLM projection for int8 decoding, before pruning/quantization: W 11008x4096 fp32 ~N(0, 0.02^2)
    (seed 37); X 4096x64 fp32 ~N(0,1) (seed 38), of which the first N columns (tokens) are used."""
    return dict(W_f32=normal_f32(37, (11008, 4096), 0.02), X_f32=normal_f32(38, (4096, 64)))


def bert_ffn_biases():
    """Biases of the BERT-base FFN pair for the fused chain: b1 (3072, seed 25), b2 (768, seed 26),
    fp32 ~N(0, 0.02^2)."""
    return dict(b1=normal_f32(25, (3072,), 0.02), b2=normal_f32(26, (768,), 0.02))


def llm_proj(M: int):
    """LLM projection, Wanda scoring: W Mx4096 bf16 ~N(0, 0.02^2) (seed 31 for M=11008, 32 for 4096);
    calibration X 4096x2048 heavy-tailed (seed 33); GEMM activations 4096x4096 same law (seed 34),
    of which the first N columns are used."""
    seed = {11008: 31, 4096: 32}[M]
    return dict(W_bf16=normal_bf16(seed, (M, 4096), 0.02), Xcal_bf16=heavy_tailed_bf16(33, 4096, 2048),
                X_bf16=heavy_tailed_bf16(34, 4096, 4096))


def ffn_28672x8192(n_max: int = 8192):
    """Large FFN: W 28672x8192 bf16 ~N(0, 0.02^2) (seed 41); X 8192 x n_max bf16 ~N(0,1) (seed 42;
    the first N columns of the 8192-wide draw are used)."""
    X = normal_f32(42, (8192, 8192))[:, :n_max]
    return dict(W_bf16=normal_bf16(41, (28672, 8192), 0.02), X_bf16=f32_to_bf16_bits(np.ascontiguousarray(X)))
