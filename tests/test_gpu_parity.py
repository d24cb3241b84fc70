"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element by element, on seeded
inputs that span several tiles with ragged tails, plus edge cases (ties, signed zeros, infinities,
N = 1 with unit row pitch, padded row pitches, K not a multiple of the instruction depth).

Bars: prune/compress/metadata/decompress and the int8 GEMM bit-exact; column norms within 1e-5
relative (double accumulation on both sides, so they are normally identical); bf16 GEMM with fp32
output within 1e-3 Frobenius relative error of the oracle's fp64 product and inside the worst-case
fp32 summation bound element by element; bf16 output equal to the kernel's own fp32 result rounded
to nearest even and within 1e-3 Frobenius of the exact product rounded to bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import (bf16_to_f64, dev, fp32_sum_bound, frob_rel, host_bits, require_gpu, rne_bf16_from_f64,
                            say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ----------------------------------------------------------------------------- inputs

def weights_f32(seed, M, K):
    """N(0, 0.02^2) rows mixed with tie-heavy rows, signed zeros and infinities."""
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    alphabet = np.array([-0.5, -0.25, -0.0, 0.0, 0.25, 0.5, 0.03125], dtype=np.float32)
    tie_rows = rng.random(M) < 0.3
    W[tie_rows] = alphabet[rng.integers(0, len(alphabet), size=(int(tie_rows.sum()), K))]
    if M > 2 and K >= 16:
        W[1, :8] = [np.inf, -np.inf, 1.0, -0.0, 0.0, -0.0, 0.0, -0.0]
    return W


def as_dtype(Wf, dt):
    if dt == "bf16":
        return synth.f32_to_bf16_bits(Wf), oracle.BF16, "bf16"
    if dt == "fp16":
        return Wf.astype(np.float16).view(np.uint16), oracle.FP16, "fp16"
    if dt in ("fp32", "fp32->bf16"):
        return Wf, oracle.FP32, None
    if dt == "i8":
        q = np.clip(np.rint(np.nan_to_num(Wf, posinf=127 / 16, neginf=-128 / 16) * 16), -128, 127)
        return q.astype(np.int8), oracle.I8, None
    raise ValueError(dt)


def padded(a, ld):
    """Copy rows into a wider buffer (row pitch ld) filled with NaN-like garbage, return the view."""
    M, K = a.shape
    buf = np.empty((M, ld), a.dtype)
    buf.view(np.uint8)[:] = 0xFF
    buf[:, :K] = a
    return buf


def wanda_norms(seed, K):
    rng = np.random.default_rng(seed)
    n = (np.exp(rng.standard_normal(K)) * 10).astype(np.float32)
    n[::5] = n[0]  # repeated norms -> score ties
    n[3] = 0.0
    return n


# ----------------------------------------------------------------------------- prune / compress


def test_prune_wanda_norms_must_be_16_byte_aligned():
    # the kernel reads the norms of a group of four as one 16-byte load: other alignments are refused
    M, K = 48, 320
    W, _, kind = as_dtype(weights_f32(7, M, K), "bf16")
    say("prune_compress wanda norms one float into their buffer")
    nbuf = dev(np.concatenate([[np.float32(1.0)], wanda_norms(K + 1, K)]).astype(np.float32))
    with pytest.raises(sp.Sp24Error) as e:
        sp.sp24_prune_compress(dev(W, kind), score=sp.SP24_SCORE_WANDA, norms=nbuf[1:])
    assert e.value.status == sp.SP24_ERR_ALIGN


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32", "fp32->bf16", "i8"])
@pytest.mark.parametrize("score", ["magnitude", "wanda"])
@pytest.mark.parametrize("M,K,ld", [(1, 16, 16), (37, 48, 64), (200, 336, 352), (3, 1024, 1024)])
def test_prune_compress_bit_exact(dt, score, M, K, ld):
    Wf = weights_f32(M * 7 + K, M, K)
    if dt == "i8" and score == "wanda":
        # Wanda scores float weights; the library refuses int8 with it, before any launch
        W8 = np.clip(np.rint(Wf * 50), -127, 127).astype(np.int8)
        with pytest.raises(sp.Sp24Error) as e:
            sp.sp24_prune_compress(dev(W8), score=sp.SP24_SCORE_WANDA, norms=dev(wanda_norms(K, K)))
        assert e.value.status == sp.SP24_ERR_DTYPE
        return
    W, odt, kind = as_dtype(Wf, dt)
    vdt = oracle.BF16 if dt == "fp32->bf16" else odt
    norms = wanda_norms(K, K) if score == "wanda" else None
    osc = oracle.WANDA if score == "wanda" else oracle.MAGNITUDE
    ref_v, ref_m = oracle.prune_compress(W, odt, osc, norms, vdt)
    Wp = padded(W, ld)
    say(f"prune_compress dt={dt} score={score} M={M} K={K} ld={ld}")
    Wd = dev(Wp, kind)[:, :K]
    val_dtype = torch.bfloat16 if dt == "fp32->bf16" else None
    vals, meta = sp.sp24_prune_compress(Wd, score=osc, norms=dev(norms) if norms is not None else None,
                                        val_dtype=val_dtype)
    torch.cuda.synchronize()
    # whole buffers, padding included, in the tiled layout
    assert np.array_equal(host_bits(meta), ref_m)
    assert np.array_equal(host_bits(vals).view(ref_v.dtype), ref_v)


_TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32, "i8": torch.int8}
_SIZE = {"bf16": 2, "fp16": 2, "fp32": 4, "i8": 1}


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32", "i8"])
def test_decompress_bit_exact_with_row_pitch(dt):
    M, K, ld = 45, 208, 240
    Wf = weights_f32(99, M, K)
    W, odt, kind = as_dtype(Wf, dt)
    v, m = oracle.prune_compress(W, odt)
    ref = oracle.decompress(v, m, odt, M, K)
    say(f"decompress dt={dt}")
    vd = dev(v, kind)
    raw = torch.full((M * ld * _SIZE[dt],), 0xFF, dtype=torch.uint8, device="cuda")
    out_buf = raw.view(_TORCH_DT[dt]).view(M, ld)
    sp.sp24_decompress(vd, dev(m), M, K, out=out_buf[:, :K])
    torch.cuda.synchronize()
    got = host_bits(out_buf)
    assert np.array_equal(got[:, :K].view(ref.dtype), ref)
    assert np.all(host_bits(out_buf[:, K:].contiguous()).view(np.uint8) == 0xFF)  # padding untouched
    # the GPU pair round-trips: decompress(compress(W)) == prune(W)
    vals, meta = sp.sp24_prune_compress(dev(W, kind))
    assert np.array_equal(host_bits(sp.sp24_decompress(vals, meta, M, K)).view(ref.dtype), ref)


# ----------------------------------------------------------------------------- column norms

@pytest.mark.parametrize("K,N,ldx", [(5, 1, 1), (7, 9, 9), (64, 2048, 2048), (33, 100, 104), (17, 777, 800),
                                     (3, 5000, 5000)])
def test_col_norms(K, N, ldx):
    X = synth.heavy_tailed_bf16(K * 31 + N, K, N)
    ref = oracle.col_norms(X)
    say(f"col_norms K={K} N={N} ldx={ldx}")
    Xp = padded(X, ldx)
    Xd = dev(Xp, "bf16")[:, :N]
    got = host_bits(sp.sp24_col_norms(Xd))
    rel = np.abs(got.astype(np.float64) - ref) / np.maximum(ref, 1e-30)
    assert rel.max() <= 1e-5
    assert np.mean(got == ref) >= 0.99  # both accumulate in double


def test_col_norms_closed_form():
    k = 5
    N = 4 ** k
    X = np.full((4, N), 0x4000, np.uint16)  # 2.0 in bf16
    X[1] = 0xC000  # -2.0
    X[2] = 0x3E80  # 0.25
    X[3] = 0
    say("col_norms closed form")
    got = host_bits(sp.sp24_col_norms(dev(X, "bf16")))
    assert got.tolist() == [2.0 * 2 ** k, 2.0 * 2 ** k, 0.25 * 2 ** k, 0.0]


# ----------------------------------------------------------------------------- sparse GEMM, bf16

GEMM_SHAPES = [
    # M, K, N, ldx, ldy
    (16, 16, 1, 1, 1),
    (16, 64, 16, 16, 16),
    (33, 48, 17, 17, 17),
    (64, 64, 64, 64, 64),
    (200, 336, 100, 104, 100),
    (300, 1024, 300, 304, 320),
    (129, 256, 1, 1, 1),
    (70, 512, 8, 8, 8),
    (256, 256, 64, 64, 64),
    (512, 768, 520, 520, 520),
    # few-token kernel (N <= 64): 1, 2 and 4 row blocks per workgroup (M >= 8192 and >= 16384 rows),
    # one to four 16-column fragments, the unit-pitch vector, a strided vector, one tile of K, K tails
    (9000, 80, 1, 1, 1),
    (600, 4096, 1, 3, 1),
    (8200, 256, 5, 5, 5),
    (16400, 128, 24, 32, 24),
    (16400, 192, 40, 40, 40),
    (100, 16, 33, 40, 33),
    (1040, 1088, 64, 64, 64),
    (2000, 208, 16, 16, 16),
    (300, 320, 8, 16, 8),
    (12000, 4096, 1, 1, 1),
    # tiled kernel (K % 64 == 0, N > 64): ragged M and N, several tiles, padded pitches
    (1000, 512, 777, 784, 777),
    (64, 64, 65, 72, 65),
    (257, 128, 513, 520, 516),
    (768, 1024, 1024, 1024, 1024),
    (40, 192, 300, 304, 300),
    # 153 tiles of 256 x 256: several turns of 256 x 128 tiles, two workgroups per CU
    (2304, 128, 4100, 4104, 4100),
]


def _gemm_inputs(M, K, N, seed):
    W = synth.normal_bf16(seed, (M, K), 0.02)
    X = synth.normal_bf16(seed + 1, (K, N))
    v, m = oracle.prune_compress(W, oracle.BF16)
    return W, X, v, m


def _check_bf16_gemm(v, m, M, X, Yf32, Ybf16, rows=None):
    Y64 = oracle.gemm_bf16(v, m, X, M, rows=rows)
    dense = bf16_to_f64(oracle.decompress(v, m, oracle.BF16, M, X.shape[0]))
    if rows is not None:
        dense = dense[rows]
    K = dense.shape[1]
    bound = fp32_sum_bound(np.abs(dense) @ np.abs(bf16_to_f64(X)), K)
    err = np.abs(Yf32.astype(np.float64) - Y64)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound)}"
    rel = frob_rel(Yf32, Y64)
    assert rel <= 1e-3, rel
    if Ybf16 is not None:
        # bf16 output = the same kernel's fp32 result rounded to nearest even ...
        assert np.array_equal(Ybf16, synth.f32_to_bf16_bits(Yf32))
        # ... and close to the exact product rounded to bf16
        assert frob_rel(bf16_to_f64(Ybf16), bf16_to_f64(rne_bf16_from_f64(Y64))) <= 1e-3
    return rel


@pytest.mark.parametrize("M,K,N,ldx,ldy", GEMM_SHAPES)
def test_gemm_bf16_parity(M, K, N, ldx, ldy):
    W, X, v, m = _gemm_inputs(M, K, N, M + K + N)
    say(f"gemm_bf16 M={M} K={K} N={N} ldx={ldx} ldy={ldy}")
    Xd = dev(padded(X, ldx), "bf16")[:, :N]
    vd, md = dev(v, "bf16"), dev(m)
    Yf = torch.full((M, ldy), 12345.0, dtype=torch.float32, device="cuda")
    Yb = torch.full((M, ldy), 12345.0, dtype=torch.bfloat16, device="cuda")
    sp.sp24_gemm_bf16(vd, md, M, Xd, out=Yf[:, :N])
    sp.sp24_gemm_bf16(vd, md, M, Xd, out=Yb[:, :N])
    torch.cuda.synchronize()
    yf, yb = host_bits(Yf), host_bits(Yb)
    assert np.all(yf[:, N:] == 12345.0)  # nothing written past N (X's padding there is NaN)
    _check_bf16_gemm(v, m, M, X, yf[:, :N], yb[:, :N])


def test_gemm_bf16_identity_equals_decompress():
    M, K = 96, 128
    W = synth.normal_bf16(3, (M, K))
    v, m = oracle.prune_compress(W, oracle.BF16)
    eye = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    say("gemm_bf16 identity")
    Y = host_bits(sp.sp24_gemm_bf16(dev(v, "bf16"), dev(m), M, dev(eye, "bf16")))
    dense = bf16_to_f64(oracle.decompress(v, m, oracle.BF16, M, K)).astype(np.float32)
    assert np.array_equal(Y, dense)


def test_gemm_bf16_orin7_gather_example():
    # Orin NN design ch. 7 sec. 2.1 Step 3: values [-0.5, 0.2] at positions {1, 3} meet x1 and x3
    W = np.zeros((1, 16), np.float32)
    W[0, 1], W[0, 3] = -0.5, 0.2
    Wb = synth.f32_to_bf16_bits(W)
    v, m = oracle.prune_compress(Wb, oracle.BF16)
    assert m[0] & 0xF == 0xD  # row 0, group 0 sits at byte 0 of the metadata
    X = synth.f32_to_bf16_bits(np.arange(1, 17, dtype=np.float32).reshape(16, 1))
    say("gemm_bf16 gather example")
    Y = host_bits(sp.sp24_gemm_bf16(dev(v, "bf16"), dev(m), 1, dev(X, "bf16")))
    x = bf16_to_f64(X[:, 0])
    assert Y[0, 0] == np.float32(bf16_to_f64(v[0]) * x[1] + bf16_to_f64(v[1]) * x[3])


# ----------------------------------------------------------------------------- sparse GEMM, int8

I8_SHAPES = [(16, 16, 1, 1), (33, 48, 17, 20), (64, 128, 64, 64), (200, 336, 100, 112), (96, 1024, 300, 304),
             (80, 512, 8, 8),
             # tiled kernel (N > 64, 16-byte X rows): ragged M and N, K tails, several tiles both ways
             (257, 512, 513, 528), (40, 128, 65, 80), (520, 1168, 1000, 1008), (300, 3072, 600, 608)]


@pytest.mark.parametrize("M,K,N,ldx", I8_SHAPES)
def test_gemm_i8_bit_exact(M, K, N, ldx):
    rng = np.random.default_rng(M * K + N)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(K, N), dtype=np.int8)
    scale = (rng.random(M) * 1e-3 + 1e-5).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    acc, Y = oracle.gemm_i8(v, m, X, M, scale)
    say(f"gemm_i8 M={M} K={K} N={N} ldx={ldx}")
    vd, md, Xd = dev(v), dev(m), dev(padded(X, ldx))[:, :N]
    got_acc = host_bits(sp.sp24_gemm_i8(vd, md, M, Xd))
    got_y = host_bits(sp.sp24_gemm_i8(vd, md, M, Xd, scale=dev(scale)))
    assert np.array_equal(got_acc.astype(np.int64), acc)
    assert np.array_equal(got_y.view(np.uint32), Y.view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(4000, 256, 4000), (3000, 640, 7000)])
def test_gemm_i8_feature_major_tile_widths_sampled(M, K, N):
    # Feature-major launches at both int8 tile widths, ragged in M and N, compared bit for bit on sampled
    # rows: 4000 x 4000 has 16 x 16 = 256 tiles of 256 x 256 (one full turn: the 256-wide tile), and
    # 3000 x 7000 has 12 x 28 = 336 of them, where 12 x 55 = 660 tiles of 256 x 128 fill three turns of
    # the cheaper tile better than two turns of 256 x 256 (the 128-wide tile, 128-byte B rows).
    rng = np.random.default_rng(M + K + N)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(K, N), dtype=np.int8)
    scale = (rng.random(M) * 1e-3 + 1e-5).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), [0, 255, 256, M - 1]]))
    acc, Y = oracle.gemm_i8(v, m, X, M, scale, rows=rows)
    say(f"gemm_i8 feature-major tile widths M={M} K={K} N={N}")
    vd, md, Xd = dev(v), dev(m), dev(X)
    r = torch.from_numpy(rows).cuda()
    got_acc = host_bits(sp.sp24_gemm_i8(vd, md, M, Xd)[r])
    got_y = host_bits(sp.sp24_gemm_i8(vd, md, M, Xd, scale=dev(scale))[r])
    assert np.array_equal(got_acc.astype(np.int64), acc)
    assert np.array_equal(got_y.view(np.uint32), Y.view(np.uint32))
