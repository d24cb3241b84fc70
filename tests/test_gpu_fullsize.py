"""GPU parity at the full sizes of the benchmark workloads, through the same C-ABI calls (hence the same
kernels and launch configurations) that bench.py times.

Every selection-type result is compared whole: prune/compress values and metadata bit-exact (the full
compressed buffers, padding included), column norms within 1e-5. GEMM outputs are compared on a
seeded sample of rows that the oracle computes one by one (fp64 for bf16, exact int64 for int8), at
every token count the workloads use: fp32 output within the fp32 summation bound element by element
and 1e-3 Frobenius; bf16 output equal to the kernel's own fp32 result rounded to nearest even; int8
output bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import bf16_to_f64, dev, fp32_sum_bound, frob_rel, host_bits, require_gpu, say
from tests.layout_ref import to_row_major

pytestmark = pytest.mark.gpu

ROWS = 48  # random output rows per GEMM, on top of one row in every 256-row block


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rows(M, seed):
    """Seeded sample of output rows: one in every 256-row block (a seeded offset inside it), so that every
    row block of the tiled kernels' 256-row tiles is checked across all N columns (hence every tile), plus
    ROWS random rows and the first and last row."""
    rng = np.random.default_rng(seed)
    r = np.sort(rng.choice(M, size=min(ROWS, M), replace=False))
    starts = np.arange(0, M, 256)
    per_block = np.minimum(starts + rng.integers(0, 256, size=len(starts)), M - 1)
    return np.unique(np.concatenate([r, per_block, [0, M - 1]]))


def _prune_bit_exact(W_host, dt, score=oracle.MAGNITUDE, norms=None, val_dtype=None):
    """Prune on both sides; returns the oracle's (values, meta) after checking the GPU's bit for bit."""
    kind = "bf16" if dt == oracle.BF16 else None
    vdt = {oracle.BF16: torch.bfloat16, oracle.FP32: torch.float32, oracle.I8: torch.int8}[dt if val_dtype is None else val_dtype]
    v, m = sp.sp24_prune_compress(dev(W_host, kind), score=score,
                                  norms=None if norms is None else dev(norms), val_dtype=vdt)
    rv, rm = oracle.prune_compress(W_host, dt, score, norms, val_dtype)
    assert np.array_equal(host_bits(m), rm)
    assert np.array_equal(host_bits(v).view(np.uint8), rv.view(np.uint8))  # bit patterns (-0, NaN-safe)
    return v, m, rv, rm


def _check_bf16(vd, md, rv, rm, M, X_host, rows):
    """Both layouts against the oracle's sampled rows: feature-major (X K x N, Y M x N) and token-major
    (X N x K, Y N x M: the sampled rows are columns of Y), the layout bench.py times by default."""
    K, N = X_host.shape
    r = torch.from_numpy(rows).cuda()
    Y64 = oracle.gemm_bf16(rv, rm, X_host, M, rows=rows)
    dense = bf16_to_f64(oracle.decompress(rv, rm, oracle.BF16, M, K)[rows])
    bound = fp32_sum_bound(np.abs(dense) @ np.abs(bf16_to_f64(X_host)), K)
    for layout in ("feature", "token"):
        if layout == "feature":
            Xd = dev(X_host, "bf16")
            pick = lambda Y: Y[r]
        else:
            Xd = dev(np.ascontiguousarray(X_host.T), "bf16")
            pick = lambda Y: Y[:, r].t().contiguous()
        Yf = host_bits(pick(sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout=layout, out_dtype=torch.float32)))
        Yb = host_bits(pick(sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout=layout, out_dtype=torch.bfloat16)))
        assert np.all(np.abs(Yf.astype(np.float64) - Y64) <= bound), layout
        assert frob_rel(Yf, Y64) <= 1e-3, layout
        assert np.array_equal(Yb, synth.f32_to_bf16_bits(Yf)), layout
        del Xd


def test_single_linear_256():
    d = synth.single_linear_256()
    say("full size: single linear 256 (fp32 prune, bf16 values, N = 64)")
    _prune_bit_exact(d["W_f32"], oracle.FP32)  # fp32 values, bit copies
    vd, md, rv, rm = _prune_bit_exact(d["W_f32"], oracle.FP32, val_dtype=oracle.BF16)
    _check_bf16(vd, md, rv, rm, 256, d["X_bf16"], np.arange(256))


def test_vit_b16_fc1():
    d = synth.vit_b16_fc1()
    say("full size: ViT-B/16 fc1 3072 x 768, N = 6304")
    vd, md, rv, rm = _prune_bit_exact(d["W_bf16"], oracle.BF16)
    _check_bf16(vd, md, rv, rm, 3072, d["X_bf16"], _rows(3072, 1))


def test_bert_ffn_int8():
    d = synth.bert_ffn_int8_dense()
    for wk, xk, seed in (("W1_f32", "X1_f32", 2), ("W2_f32", "X2_f32", 3)):
        W = d[wk]
        M, K = W.shape
        say(f"full size: BERT FFN int8 {M} x {K}, N = 8192")
        # fp32 prune (GPU bit-exact with the oracle), then the host int8 preparation from the oracle's
        # pruned weight, then the int8 prune/compress (bit-exact) and the int8 GEMM (bit-exact)
        _, _, rv, rm = _prune_bit_exact(W, oracle.FP32)
        Wp = oracle.decompress(rv, rm, oracle.FP32, M, K)
        q, s_w = synth.quantize_rows(Wp)
        xq, s_x = synth.quantize_tensor(d[xk])
        scale = synth.dequant_scales(s_w, s_x)
        v8, m8, rv8, rm8 = _prune_bit_exact(q, oracle.I8)
        rows = _rows(M, seed)
        r = torch.from_numpy(rows).cuda()
        Xd = dev(xq)
        got = host_bits(sp.sp24_gemm_i8(v8, m8, M, Xd, scale=dev(scale))[r])
        got_acc = host_bits(sp.sp24_gemm_i8(v8, m8, M, Xd)[r])
        acc, Y = oracle.gemm_i8(rv8, rm8, xq, M, scale, rows=rows)
        assert np.array_equal(got_acc.astype(np.int64), acc)
        assert np.array_equal(got.view(np.uint32), Y.view(np.uint32))
        # token-major (X N x K, Y N x M), the layout the bench times
        Xt = dev(np.ascontiguousarray(xq.T))
        got_tm = host_bits(sp.sp24_gemm_i8_ex(v8, m8, M, Xt, scale=dev(scale), layout="token")[:, r].t().contiguous())
        assert np.array_equal(got_tm.view(np.uint32), Y.view(np.uint32))


def test_llm_projection_int8_few_tokens():
    # the int8 decode workload: fp32 prune (bit-exact), host int8 preparation from the oracle's pruned
    # weight, int8 prune/compress (bit-exact), then the few-token int8 GEMM token-major (bit-exact on
    # sampled rows, int32 and fp32 output) at N = 1, 16 and 64
    d = synth.llm_proj_int8_dense()
    W = d["W_f32"]
    M, K = W.shape
    say(f"full size: LLM projection int8 {M} x {K}, N in 1, 16, 64")
    _, _, rv, rm = _prune_bit_exact(W, oracle.FP32)
    q, s_w = synth.quantize_rows(oracle.decompress(rv, rm, oracle.FP32, M, K))
    v8, m8, rv8, rm8 = _prune_bit_exact(q, oracle.I8)
    rows = _rows(M, 6)
    r = torch.from_numpy(rows).cuda()
    for N in (1, 16, 64):
        xq, s_x = synth.quantize_tensor(np.ascontiguousarray(d["X_f32"][:, :N]))
        scale = synth.dequant_scales(s_w, s_x)
        acc, Y = oracle.gemm_i8(rv8, rm8, xq, M, scale, rows=rows)
        Xt = dev(np.ascontiguousarray(xq.T))
        got = host_bits(sp.sp24_gemm_i8_ex(v8, m8, M, Xt, scale=dev(scale), layout="token")[:, r].t().contiguous())
        got_acc = host_bits(sp.sp24_gemm_i8_ex(v8, m8, M, Xt, layout="token")[:, r].t().contiguous())
        assert np.array_equal(got_acc.astype(np.int64), acc)
        assert np.array_equal(got.view(np.uint32), Y.view(np.uint32))


@pytest.mark.parametrize("M", [11008, 4096])
def test_llm_projection_wanda(M):
    d = synth.llm_proj(M)
    say(f"full size: LLM projection {M} x 4096 with Wanda, N in 1, 16, 4096")
    norms = host_bits(sp.sp24_col_norms(dev(d["Xcal_bf16"], "bf16")))
    ref_norms = oracle.col_norms(d["Xcal_bf16"])
    assert np.max(np.abs(norms.astype(np.float64) - ref_norms) / ref_norms) <= 1e-5
    # prune with the oracle's norms on both sides, so the selection compares bit for bit
    vd, md, rv, rm = _prune_bit_exact(d["W_bf16"], oracle.BF16, oracle.WANDA, ref_norms)
    rows = _rows(M, 4)
    for N in (1, 16, 4096):
        _check_bf16(vd, md, rv, rm, M, np.ascontiguousarray(d["X_bf16"][:, :N]), rows)


def _nibbles(values, meta, M, K):
    """Row-major group nibbles (M x K/4) of a bf16 compressed weight."""
    _, m = to_row_major(values, meta, M, K, 2)
    m = m.astype(np.uint8)
    return np.stack([m & 0xF, m >> 4], axis=2).reshape(M, K // 4)


@pytest.mark.parametrize("M", [11008, 4096])
def test_llm_projection_wanda_chain(M):
    """The chain bench.py times, GPU column norms then GPU Wanda prune, against the oracle's chain (oracle
    norms, oracle prune). Given the same norms the prune is bit-exact; the GPU norms may differ from the
    oracle's in the last bits (within 1e-5 relative), so a group may keep a different pair only where a kept
    and a dropped score lie within that tolerance of each other. Such groups are counted and bounded."""
    d = synth.llm_proj(M)
    W, Xcal = d["W_bf16"], d["Xcal_bf16"]
    K = W.shape[1]
    say(f"full size: Wanda chain {M} x {K}, GPU norms -> GPU prune against the oracle chain")
    gn = host_bits(sp.sp24_col_norms(dev(Xcal, "bf16")))
    on = oracle.col_norms(Xcal)
    rel = np.abs(gn.astype(np.float64) - on) / on
    assert np.max(rel) <= 1e-5
    v_g, m_g = sp.sp24_prune_compress(dev(W, "bf16"), score=sp.SP24_SCORE_WANDA, norms=dev(gn))
    v_g, m_g = host_bits(v_g), host_bits(m_g)
    # the GPU prune with the GPU norms is the oracle's prune with the same norms, bit for bit
    rv_gn, rm_gn = oracle.prune_compress(W, oracle.BF16, oracle.WANDA, gn)
    assert np.array_equal(m_g, rm_gn) and np.array_equal(v_g, rv_gn)
    # against the oracle's whole chain
    rv, rm = oracle.prune_compress(W, oracle.BF16, oracle.WANDA, on)
    ng, no = _nibbles(v_g, m_g, M, K), _nibbles(rv, rm, M, K)
    diff = np.argwhere(ng != no)
    # scores under the oracle's norms: fl32(fl32(|w|) * norm)
    a = np.abs(bf16_to_f64(W).astype(np.float32))
    for i, g in diff:
        s = (a[i, 4 * g:4 * g + 4] * on[4 * g:4 * g + 4]).astype(np.float64)
        kg = {int(ng[i, g]) & 3, int(ng[i, g]) >> 2}
        ko = {int(no[i, g]) & 3, int(no[i, g]) >> 2}
        (x,), (y,) = kg - ko, ko - kg  # kept only by the GPU chain, kept only by the oracle chain
        assert abs(s[x] - s[y]) <= 3e-5 * max(s[x], s[y]), (i, g, s)
    frac = len(diff) / (M * K / 4)
    say(f"Wanda chain {M} x {K}: {len(diff)} of {M * K // 4} groups differ (near-ties of the norms), {frac:.2e}")
    assert frac <= 1e-4


def test_ffn_28672x8192():
    d = synth.ffn_28672x8192(8192)
    say("full size: FFN 28672 x 8192, N in 8, 64, 512, 8192")
    vd, md, rv, rm = _prune_bit_exact(d["W_bf16"], oracle.BF16)
    # the first 1024 rows whole (the slice the CPU baseline times) and 256 more: one in every 256-row
    # tile row, the rest at random
    rng = np.random.default_rng(5)
    per_block = np.arange(0, 28672, 256) + rng.integers(0, 256, size=112)
    extra = rng.choice(np.arange(1024, 28672), size=256, replace=False)
    rows = np.unique(np.concatenate([np.arange(1024), per_block, extra, [28671]]))
    assert len(np.unique(rows // 256)) == 112 and np.all(rows[:1024] == np.arange(1024))  # every tile row
    for N in (8, 64, 512, 8192):
        _check_bf16(vd, md, rv, rm, 28672, np.ascontiguousarray(d["X_bf16"][:, :N]), rows)


def test_ffn_one_gpu_share():
    """Rows [0, 3584) of the FFN weight: one GPU's share of an output-channel split over eight GPUs, the shape
    `bench.py --shard-m 8` times (other kernels' launch configurations than the whole layer at N = 8)."""
    d = synth.ffn_28672x8192(8192)
    W = np.ascontiguousarray(d["W_bf16"][:3584])
    say("full size: FFN one-GPU share 3584 x 8192, N in 8, 8192")
    vd, md, rv, rm = _prune_bit_exact(W, oracle.BF16)
    rows = _rows(3584, 8)
    assert len(np.unique(rows // 256)) == 14
    for N in (8, 8192):
        _check_bf16(vd, md, rv, rm, 3584, np.ascontiguousarray(d["X_bf16"][:, :N]), rows)


def test_bert_ffn_int8_fused_chain():
    # the fused chain the bench times (token-major): H = int8(GELU(W1 X + b1)), Y = W2 H + b2
    d = synth.bert_ffn_int8_dense()
    bias = synth.bert_ffn_biases()
    qs = []
    for wk in ("W1_f32", "W2_f32"):
        W = d[wk]
        M, K = W.shape
        _, _, rv, rm = _prune_bit_exact(W, oracle.FP32)
        qs.append(synth.quantize_rows(oracle.decompress(rv, rm, oracle.FP32, M, K)))
    (q1, s_w1), (q2, s_w2) = qs
    xq, s_x = synth.quantize_tensor(d["X1_f32"])
    Xt = np.ascontiguousarray(xq.T)  # 8192 tokens x 768
    s1 = synth.dequant_scales(s_w1, s_x)
    s_h = 0.01  # a fixed hidden scale (the codes' range is what matters here)
    s2 = synth.dequant_scales(s_w2, np.float32(s_h))
    say("full size: BERT FFN int8 fused chain, token-major, N = 8192")
    v1, m1, rv1, rm1 = _prune_bit_exact(q1, oracle.I8)
    v2, m2, rv2, rm2 = _prune_bit_exact(q2, oracle.I8)
    H = sp.sp24_gemm_i8_fused(v1, m1, 3072, dev(Xt), dev(s1), bias=dev(bias["b1"]), activation="gelu",
                              out_dtype=torch.int8, out_scale=s_h, layout="token")
    Y = sp.sp24_gemm_i8_fused(v2, m2, 768, H, dev(s2), bias=dev(bias["b2"]), layout="token")
    rows = _rows(3072, 6)
    h = host_bits(H)
    ref = oracle.gemm_i8_fused(rv1, rm1, Xt, 3072, s1, bias["b1"], gelu=True, out_scale=s_h, rows=rows,
                               layout="token")
    got = h[:, rows].astype(np.int32)
    assert np.all(np.abs(got - ref["q"].astype(np.int32)) <= 1)
    assert np.mean(got == ref["q"]) > 0.999
    # GEMM 2 is bit-exact on the codes the GPU produced
    rows2 = _rows(768, 7)
    y = host_bits(Y)[:, rows2]
    ref2 = oracle.gemm_i8_fused(rv2, rm2, h, 768, s2, bias["b2"], rows=rows2, layout="token")["y"]
    assert np.array_equal(y.view(np.uint32), ref2.view(np.uint32))
