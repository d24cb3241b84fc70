"""GPU parity of the input-channel permutation search (sp24_channel_permutation; Orin NN design,
Chapter 7, section 3.1 Step 2 and section 6.3). The search is deterministic and both sides sum the
objective in double precision in the same order, so the GPU's permutation must equal the oracle's
exactly; it must also be a permutation whose retained score is at least the unpermuted one, and the
pruned product with the permuted weight and permuted activations is the same computation."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import bf16_to_f64, dev, frob_rel, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu

_KIND = {oracle.BF16: "bf16", oracle.FP16: "fp16", oracle.FP32: None, oracle.I8: None}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _weight(dt, M, K, seed):
    rng = np.random.default_rng(seed)
    if dt == oracle.I8:
        return rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    x = (rng.standard_normal((M, K)) * rng.lognormal(0, 1, K)[None, :]).astype(np.float32)
    if dt == oracle.FP32:
        return x
    if dt == oracle.FP16:
        return x.astype(np.float16).view(np.uint16)
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dt,M,K,ld,sweeps", [
    (oracle.BF16, 64, 64, 64, 1),
    (oracle.BF16, 300, 104, 112, 2),   # rows past one LDS block, 26 groups
    (oracle.FP16, 37, 20, 24, 3),      # 5 groups: one sits out each round
    (oracle.FP32, 129, 96, 96, 1),
    (oracle.I8, 200, 128, 144, 2),
    (oracle.BF16, 16, 8, 8, 1),        # one pair: the best of its 35 splits
])
def test_permutation_matches_oracle(dt, M, K, ld, sweeps):
    W = _weight(dt, M, K, M * K + sweeps)
    say(f"channel_permutation dt={dt} M={M} K={K} ld={ld} sweeps={sweeps}")
    Wp = np.zeros((M, ld), W.dtype)
    Wp[:, :K] = W
    perm = host_bits(sp.sp24_channel_permutation(dev(Wp, _KIND[dt])[:, :K], sweeps))
    ref = oracle.channel_permutation(W, dt, sweeps)
    assert np.array_equal(perm, ref)
    assert sorted(perm.tolist()) == list(range(K))
    assert oracle.retained(W, dt, perm) >= oracle.retained(W, dt)


def test_permutation_wanda_matches_oracle():
    M, K = 96, 128
    W = _weight(oracle.BF16, M, K, 5)
    norms = np.abs(np.random.default_rng(6).standard_normal(K)).astype(np.float32) + 0.05
    say("channel_permutation wanda")
    perm = host_bits(sp.sp24_channel_permutation(dev(W, "bf16"), 2, score=sp.SP24_SCORE_WANDA, norms=dev(norms)))
    ref = oracle.channel_permutation(W, oracle.BF16, 2, oracle.WANDA, norms)
    assert np.array_equal(perm, ref)


def test_permutation_full_size_vit_and_product():
    # the ViT-B/16 fc1 weight (3072 x 768), one sweep, then the pruned product with permuted X
    d = synth.vit_b16_fc1()
    W, X = d["W_bf16"], d["X_bf16"]
    say("channel_permutation full size ViT fc1, one sweep")
    Wd = dev(W, "bf16")
    perm_d = sp.sp24_channel_permutation(Wd, 1)
    perm = host_bits(perm_d)
    assert np.array_equal(perm, oracle.channel_permutation(W, oracle.BF16, 1))
    r0, r1 = oracle.retained(W, oracle.BF16), oracle.retained(W, oracle.BF16, perm)
    assert r1 > r0
    # prune the permuted weight and multiply by X with its rows in the same order: the kept weights
    # meet the same activations as in W's own column order
    Wperm = Wd[:, perm_d.long()].contiguous()
    Xperm = dev(X, "bf16")[perm_d.long(), :].contiguous()
    v, m = sp.sp24_prune_compress(Wperm)
    Y = host_bits(sp.sp24_gemm_bf16(v, m, 3072, Xperm, out_dtype=torch.float32))
    rows = np.arange(0, 3072, 97)
    rv, rm = oracle.prune_compress(np.ascontiguousarray(W[:, perm]), oracle.BF16)
    Y64 = oracle.gemm_bf16(rv, rm, np.ascontiguousarray(X[perm, :]), 3072, rows=rows)
    assert frob_rel(Y[rows], Y64) <= 1e-3
