"""GPU parity of the k-of-4 masks (sp24_prune_mask; NVIDIA blog, progressive sparse training, Figure 4):
mask nibbles and masked weights bit-exact against the oracle for every dtype, keep = 1..4, magnitude
and Wanda scores, ragged M, padded pitches, tie-heavy rows and signed zeros; and the progressive
schedule (keep 3 of 4, then 2 of 4 on the masked weight) equal to the direct 2-of-4 mask and to the
2:4 compression's positions."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import dev, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu

_KIND = {oracle.BF16: "bf16", oracle.FP16: "fp16", oracle.FP32: None, oracle.I8: None}
_NP = {oracle.BF16: np.uint16, oracle.FP16: np.uint16, oracle.FP32: np.float32, oracle.I8: np.int8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _weight(dt, M, K, seed):
    rng = np.random.default_rng(seed)
    if dt == oracle.I8:
        W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
        W[:, ::5] = W[:, 1::5][:, : W[:, ::5].shape[1]]  # repeated values: ties
        return W
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, ::6] = 0.0
    x[:, 1::9] = -0.0
    x[:, 2::11] = x[:, 3::11][:, : x[:, 2::11].shape[1]]  # equal magnitudes
    if dt == oracle.FP32:
        return x
    if dt == oracle.FP16:
        return x.astype(np.float16).view(np.uint16)
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16, oracle.FP32, oracle.I8])
@pytest.mark.parametrize("keep", [1, 2, 3, 4])
@pytest.mark.parametrize("M,K,ld", [(37, 208, 208), (300, 1024, 1040)])
def test_mask_bit_exact(dt, keep, M, K, ld):
    W = _weight(dt, M, K, M + K + keep + dt)
    say(f"prune_mask dt={dt} keep={keep} M={M} K={K} ld={ld}")
    Wp = np.zeros((M, ld), W.dtype)
    Wp[:, :K] = W
    Wd = dev(Wp, _KIND[dt])[:, :K]
    out = torch.full((M, ld), 0, dtype=Wd.dtype, device="cuda")
    out_h = host_bits(out)
    mask, _ = sp.sp24_prune_mask(Wd, keep, out=out[:, :K])
    rm, rw = oracle.prune_mask(W, dt, keep)
    assert np.array_equal(host_bits(mask), rm)
    got = host_bits(out)
    assert np.array_equal(got[:, :K].view(np.uint8), rw.view(np.uint8))
    assert np.array_equal(got[:, K:], out_h[:, K:])  # nothing written past K


@pytest.mark.parametrize("keep", [1, 2, 3])
def test_mask_wanda(keep):
    M, K = 96, 512
    W = _weight(oracle.BF16, M, K, 11)
    norms = np.abs(np.random.default_rng(12).standard_normal(K)).astype(np.float32)
    say(f"prune_mask wanda keep={keep}")
    mask, out = sp.sp24_prune_mask(dev(W, "bf16"), keep, score=sp.SP24_SCORE_WANDA, norms=dev(norms))
    rm, rw = oracle.prune_mask(W, oracle.BF16, keep, oracle.WANDA, norms)
    assert np.array_equal(host_bits(mask), rm)
    assert np.array_equal(host_bits(out), rw)


def test_progressive_schedule_equals_direct():
    M, K = 3072, 768
    W = synth.normal_bf16(13, (M, K), 0.02)
    say("prune_mask progressive 3 -> 2 of 4 at 3072 x 768")
    Wd = dev(W, "bf16")
    _, w3 = sp.sp24_prune_mask(Wd, 3)
    m2_chain, w2_chain = sp.sp24_prune_mask(w3, 2)
    m2, w2 = sp.sp24_prune_mask(Wd, 2)
    assert torch.equal(m2_chain, m2) and torch.equal(w2_chain.view(torch.int16), w2.view(torch.int16))
    # and the 2-of-4 mask is the 2:4 compression's selection
    v, m = sp.sp24_prune_compress(Wd)
    dense = sp.sp24_decompress(v, m, M, K)
    assert torch.equal(dense.view(torch.int16), w2.view(torch.int16))
    rm, _ = oracle.prune_mask(W, oracle.BF16, 2)
    assert np.array_equal(host_bits(m2), rm)
