"""GPU parity of the token-major layout (X N x K, Y N x M: a Linear layer's input and output) and of
batched products sharing one weight (a 1x1 conv over NCHW images is a batch of feature-major
products), through sp24_gemm_bf16_ex / sp24_gemm_i8_ex. Each case is compared with the oracle on the
same inputs under the bars of the feature-major tests: bf16 within the fp32 summation bound element
by element and 1e-3 Frobenius, bf16 output equal to the kernel's own fp32 result rounded to nearest
even; int8 bit-exact. Shapes reach the few-token, LDS-tiled and direct kernels, with ragged M and N,
K tails, padded pitches, and nothing written outside the output views."""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import bf16_to_f64, dev, fp32_sum_bound, frob_rel, host_bits, require_gpu, say

pytestmark = pytest.mark.gpu

SENTINEL = 12345.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _padded(a, ld, fill):
    out = np.full((a.shape[0], ld), fill, a.dtype)
    out[:, :a.shape[1]] = a
    return out


def _check_bf16(v, m, M, X_tm, yf_tm, yb_tm):
    """yf_tm / yb_tm: N x M results of the token-major product with X_tm (N x K)."""
    Y64 = oracle.gemm_bf16(v, m, X_tm, M, layout="token")  # N x M
    dense = bf16_to_f64(oracle.decompress(v, m, oracle.BF16, M, X_tm.shape[1]))
    bound = fp32_sum_bound(np.abs(bf16_to_f64(X_tm)) @ np.abs(dense).T, X_tm.shape[1])
    err = np.abs(yf_tm.astype(np.float64) - Y64)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound)}"
    assert frob_rel(yf_tm, Y64) <= 1e-3
    assert np.array_equal(yb_tm, synth.f32_to_bf16_bits(yf_tm))


TM_SHAPES = [
    # M, K, N, ldx (>= K), ldy (>= M)
    # few-token kernel: 16-byte rows, element rows (ldx % 8 != 0), K tail tiles, one token
    (16, 16, 1, 16, 16),
    (33, 48, 17, 48, 40),
    (9000, 80, 1, 80, 9000),
    (8200, 256, 5, 264, 8200),
    (16400, 128, 24, 128, 16400),
    (600, 208, 16, 208, 600),
    (300, 320, 8, 321, 304),
    (1040, 1088, 64, 1088, 1040),
    # few-token kernel with the weight streamed through LDS (N <= 2, or N <= 8 below 1024 row blocks;
    # 16-byte rows): 4, 8 and 16 waves, 2- and 8-row X tiles, K tails (80, 208, 240), one K tile per
    # wave or several; and N = 9 .. 16 on the register-pipelined kernel
    (9000, 192, 16, 200, 9000),
    # 9 to 16 tokens from 384 row blocks (the register kernel with 2, 4 or 8 row blocks per workgroup): odd
    # block counts (a last workgroup with fewer blocks), a K tail
    (16400, 240, 13, 248, 16400),
    (8200, 4096, 16, 4096, 8200),
    (6150, 320, 11, 320, 6150),
    (4400, 256, 16, 264, 4400),   # 275 row blocks: the register kernel, two blocks per workgroup
    (4096, 128, 13, 136, 4096),   # 256 row blocks: the LDS ring, one workgroup per CU
    (6150, 320, 5, 328, 6150),  # 3-8 tokens at 257-512 row blocks: the register kernel, K tail
    (9000, 256, 6, 264, 9000),  # 3-8 tokens from 513 row blocks: 4-wave ring workgroups
    # the register-pipelined few-token kernel, token-major, one round of at most one workgroup per CU (R =
    # ceil(blocks / CUs): 3, 5, 6 and 7 here, with a last workgroup holding fewer blocks), the two-block
    # workgroups several per CU, ragged block counts, a K tail
    (25000, 128, 12, 128, 25000),
    (24000, 128, 28, 136, 24000),
    (20480, 128, 16, 128, 20480),
    (17000, 208, 16, 216, 17000),
    (20000, 128, 30, 128, 20000),
    (12000, 256, 20, 264, 12000),
    (6000, 128, 24, 128, 6000),
    (3500, 128, 17, 136, 3500),
    (20000, 128, 40, 128, 20000),
    (12000, 128, 64, 128, 12000),
    (6000, 208, 48, 216, 6000),
    (4000, 320, 12, 320, 4000),
    (3100, 256, 3, 264, 3100),
    (2050, 240, 9, 248, 2056),
    (5000, 4096, 1, 4096, 5000),
    (1000, 256, 7, 256, 1000),
    (1000, 240, 2, 248, 1008),
    # LDS-tiled kernel (K % 64 == 0, N > 64): ragged M and N, padded pitches
    (1000, 512, 777, 512, 1000),
    (64, 64, 65, 72, 64),
    (257, 128, 513, 136, 260),
    (768, 1024, 1024, 1024, 768),
    (40, 192, 300, 192, 48),
    (2304, 128, 4100, 136, 2304),  # 153 tiles of 256 x 256: several turns of 256 x 128 tiles, two per CU
    # direct kernel (K tail with N > 64, or unaligned rows)
    (200, 336, 100, 336, 200),
    (96, 256, 130, 259, 97),
]


@pytest.mark.parametrize("M,K,N,ldx,ldy", TM_SHAPES)
def test_gemm_bf16_token_major(M, K, N, ldx, ldy):
    W = synth.normal_bf16(M + 3 * K, (M, K), 0.02)
    X = synth.normal_bf16(N + 5 * K, (N, K))
    v, m = oracle.prune_compress(W, oracle.BF16)
    say(f"gemm_bf16_ex token-major M={M} K={K} N={N} ldx={ldx} ldy={ldy}")
    Xd = dev(_padded(X, ldx, 0x7FC0), "bf16")[:, :K]  # NaN past K: must never be read
    vd, md = dev(v, "bf16"), dev(m)
    Yf = torch.full((N, ldy), SENTINEL, dtype=torch.float32, device="cuda")
    Yb = torch.full((N, ldy), SENTINEL, dtype=torch.bfloat16, device="cuda")
    sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout="token", out=Yf[:, :M])
    sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout="token", out=Yb[:, :M])
    yf, yb = host_bits(Yf), host_bits(Yb)
    assert np.all(yf[:, M:] == SENTINEL)
    _check_bf16(v, m, M, X, yf[:, :M], yb[:, :M])


BATCH_SHAPES = [
    # batch, M, K, N, layout -- 1x1 conv over NCHW images (feature-major, N = H*W) and batched tokens
    (3, 64, 128, 49, "feature"),
    (2, 256, 512, 196, "feature"),
    (4, 96, 80, 300, "feature"),
    (2, 128, 256, 100, "token"),
    (3, 48, 64, 20, "token"),
    (2, 300, 208, 90, "token"),
    (2, 8200, 128, 10, "token"),
    (3, 200, 320, 12, "token"),
    (2, 200, 320, 6, "token"),
]


@pytest.mark.parametrize("B,M,K,N,layout", BATCH_SHAPES)
def test_gemm_bf16_batched(B, M, K, N, layout):
    W = synth.normal_bf16(B + M + K, (M, K), 0.02)
    v, m = oracle.prune_compress(W, oracle.BF16)
    xs = [synth.normal_bf16(100 * b + N, (N, K) if layout == "token" else (K, N)) for b in range(B)]
    say(f"gemm_bf16_ex batched B={B} M={M} K={K} N={N} {layout}")
    # entries one row apart beyond their extent (strides not a multiple of the entry size)
    Xd = torch.stack([dev(x, "bf16") for x in xs] + [dev(xs[0], "bf16")])[:B]
    ysh = (N, M) if layout == "token" else (M, N)
    Yf = torch.full((B + 1,) + ysh, SENTINEL, dtype=torch.float32, device="cuda")
    Yb = torch.full((B + 1,) + ysh, SENTINEL, dtype=torch.bfloat16, device="cuda")
    sp.sp24_gemm_bf16_ex(v_d := dev(v, "bf16"), m_d := dev(m), M, Xd, layout=layout, out=Yf[:B])
    sp.sp24_gemm_bf16_ex(v_d, m_d, M, Xd, layout=layout, out=Yb[:B])
    yf, yb = host_bits(Yf), host_bits(Yb)
    assert np.all(yf[B] == SENTINEL)
    for b in range(B):
        if layout == "token":
            _check_bf16(v, m, M, xs[b], yf[b], yb[b])
        else:
            _check_bf16(v, m, M, np.ascontiguousarray(xs[b].T), np.ascontiguousarray(yf[b].T),
                        np.ascontiguousarray(yb[b].T))


def test_gemm_bf16_batched_broadcast_x():
    # x batch stride 0: every entry multiplies the same X
    M, K, N, B = 80, 128, 70, 3
    W = synth.normal_bf16(1, (M, K), 0.02)
    X = synth.normal_bf16(2, (K, N))
    v, m = oracle.prune_compress(W, oracle.BF16)
    Xd = dev(X, "bf16").unsqueeze(0).expand(B, K, N)
    say("gemm_bf16_ex batched broadcast X")
    Y = host_bits(sp.sp24_gemm_bf16_ex(dev(v, "bf16"), dev(m), M, Xd))
    for b in range(1, B):
        assert np.array_equal(Y[b], Y[0])
    _check_bf16(v, m, M, np.ascontiguousarray(X.T), np.ascontiguousarray(Y[0].T),
                synth.f32_to_bf16_bits(np.ascontiguousarray(Y[0].T)))


I8_TM_SHAPES = [
    # M, K, N, ldx (>= K), ldy (>= M): tiled (K % 128 == 0, 16-byte rows, N > 64) and direct
    (257, 512, 513, 528, 264),
    (2304, 384, 4100, 400, 2312),  # 153 tiles of 256 x 256: the 256-wide tile (smaller shapes take 128)
    (40, 128, 65, 128, 48),
    (520, 1152, 1000, 1152, 520),
    (33, 48, 17, 48, 40),
    (200, 336, 100, 336, 200),
    (96, 256, 130, 260, 97),
    # few-token int8 kernel (N <= 64, K % 128 == 0, 16-byte rows): ragged M, every fragment count
    (700, 384, 1, 384, 704),
    (1000, 256, 5, 272, 1000),
    (517, 512, 16, 512, 520),
    (300, 1024, 17, 1040, 300),
    (96, 128, 33, 144, 100),
    # few-token int8 kernel with two row blocks per workgroup (more than 1024 row blocks, or more than 512
    # with two or more fragments) and an odd block count, so the last workgroup holds one block
    (16400, 256, 1, 256, 16400),  # also the LDS-ring loop (one or two tokens from 1024 row blocks)
    (16400, 256, 20, 272, 16408),
    (16400, 256, 40, 256, 16400),
    (16400, 256, 64, 256, 16416),
    (8200, 256, 33, 256, 8200),
    # the LDS-ring loop at 9-16 tokens below 1024 row blocks: four-wave workgroups from 512 blocks (odd count),
    # eight-wave below
    (10000, 384, 13, 384, 10008),
    # LDS-ring units of three (688 row blocks) and four (894: a last workgroup of two) row blocks
    (11008, 384, 13, 384, 11016),
    (14300, 128, 9, 128, 14300),
    (16000, 256, 16, 272, 16000),
    (6000, 256, 11, 256, 6000),
    (8200, 256, 7, 272, 8200),
    # the register loop's grid sizes: more row blocks per workgroup as the weight grows (ragged block counts)
    (16400, 256, 12, 256, 16400),
    (16400, 256, 5, 256, 16408),
    (8200, 256, 24, 256, 8200),
    (6000, 256, 30, 272, 6000),
    (5000, 256, 36, 256, 5000),
    (9000, 256, 64, 256, 9000),
    (4500, 256, 50, 256, 4504),
    # one round of workgroups with R = ceil(blocks / CUs): four blocks at one fragment (1024 blocks), three
    # at three fragments (688 blocks)
    (16384, 256, 12, 256, 16384),
    (11008, 256, 40, 256, 11008),
    (33, 128, 48, 128, 36),
    (2050, 640, 64, 640, 2056),
    # 128-wide tiles with two workgroups per compute unit (token-major, more tiles than compute units):
    # 585 tiles over 512 workgroups, two stages per tile; 645 tiles, three stages; ragged M and N
    (2300, 256, 8200, 272, 2312),
    (1100, 384, 16500, 384, 1104),
]


@pytest.mark.parametrize("M,K,N,ldx,ldy", I8_TM_SHAPES)
def test_gemm_i8_token_major(M, K, N, ldx, ldy):
    rng = np.random.default_rng(M * K + N + 7)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    scale = (rng.random(M) * 1e-3 + 1e-5).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    acc, Y = oracle.gemm_i8(v, m, X, M, scale, layout="token")
    say(f"gemm_i8_ex token-major M={M} K={K} N={N} ldx={ldx} ldy={ldy}")
    Xd = dev(_padded(X, ldx, 127))[:, :K]
    vd, md = dev(v), dev(m)
    Ya = torch.full((N, ldy), -7, dtype=torch.int32, device="cuda")
    Yf = torch.full((N, ldy), SENTINEL, dtype=torch.float32, device="cuda")
    sp.sp24_gemm_i8_ex(vd, md, M, Xd, layout="token", out=Ya[:, :M])
    sp.sp24_gemm_i8_ex(vd, md, M, Xd, scale=dev(scale), layout="token", out=Yf[:, :M])
    ya, yf = host_bits(Ya), host_bits(Yf)
    assert np.all(ya[:, M:] == -7) and np.all(yf[:, M:] == SENTINEL)
    assert np.array_equal(ya[:, :M].astype(np.int64), acc)
    assert np.array_equal(yf[:, :M].view(np.uint32), Y.view(np.uint32))


@pytest.mark.parametrize("B,M,K,N,layout", [(3, 64, 256, 100, "feature"), (2, 96, 384, 80, "token"),
                                            (2, 40, 48, 30, "feature"), (3, 200, 256, 12, "token"),
                                            (2, 1100, 256, 8200, "token")])  # two workgroups per compute unit
def test_gemm_i8_batched(B, M, K, N, layout):
    rng = np.random.default_rng(B * M + K + N)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    xs = [rng.integers(-128, 128, size=(N, K) if layout == "token" else (K, N), dtype=np.int8) for _ in range(B)]
    scale = (rng.random(M) * 1e-3 + 1e-5).astype(np.float32)
    v, m = oracle.prune_compress(W, oracle.I8)
    say(f"gemm_i8_ex batched B={B} M={M} K={K} N={N} {layout}")
    Xd = torch.stack([dev(x) for x in xs])
    Y = host_bits(sp.sp24_gemm_i8_ex(dev(v), dev(m), M, Xd, scale=dev(scale), layout=layout))
    for b in range(B):
        _, ref = oracle.gemm_i8(v, m, xs[b], M, scale, layout=layout)
        assert np.array_equal(Y[b].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("layout", ["feature", "token"])
def test_gemm_bf16_many_tiles_sampled(layout):
    # 18 x 31 = 558 tiles of 256 x 256 (more than two turns of the compute units: the 256-wide tile with
    # one workgroup per CU), ragged in M and N; the oracle computes a sample of rows
    M, K, N = 4360, 192, 7900
    W = synth.normal_bf16(91, (M, K), 0.02)
    X = synth.normal_bf16(92, (K, N))
    v, m = oracle.prune_compress(W, oracle.BF16)
    rows = np.unique(np.concatenate([np.random.default_rng(93).choice(M, 40, replace=False), [0, 255, 256, M - 1]]))
    say(f"gemm_bf16_ex many tiles {layout} M={M} K={K} N={N}")
    vd, md = dev(v, "bf16"), dev(m)
    r = torch.from_numpy(rows).cuda()
    if layout == "feature":
        Xd, pick = dev(X, "bf16"), (lambda Y: Y[r])
    else:
        Xd, pick = dev(np.ascontiguousarray(X.T), "bf16"), (lambda Y: Y[:, r].t().contiguous())
    Yf = host_bits(pick(sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout=layout, out_dtype=torch.float32)))
    Yb = host_bits(pick(sp.sp24_gemm_bf16_ex(vd, md, M, Xd, layout=layout, out_dtype=torch.bfloat16)))
    Y64 = oracle.gemm_bf16(v, m, X, M, rows=rows)
    dense = bf16_to_f64(oracle.decompress(v, m, oracle.BF16, M, K)[rows])
    bound = fp32_sum_bound(np.abs(dense) @ np.abs(bf16_to_f64(X)), K)
    assert np.all(np.abs(Yf.astype(np.float64) - Y64) <= bound)
    assert frob_rel(Yf, Y64) <= 1e-3
    assert np.array_equal(Yb, synth.f32_to_bf16_bits(Yf))
