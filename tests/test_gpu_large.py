"""GPU parity where an operand passes 4 GiB, so that byte offsets need more than 32 bits: the weight and its
compressed values, the activations of either layout, and the output. One MI355X holds such operands (288 GB
of HBM), and the kernels address them through per-tile buffer bases, 64-bit pointers, or, where a 32-bit
offset could not reach, the direct kernel.

Inputs are periodic: row i of the weight is row i mod P of a small seeded block, token n of the activations is
token n mod P of another, with P prime, so that no wrap of an offset at 2^32 bytes maps an element onto an
equal one (the wrap distances in rows or tokens used here are not multiples of P). The oracle computes the
block's results once, and every row or token of the GPU's output is compared with its block row: selection,
compressed buffers, decompression and int8 products bit-exact, bf16 products within the fp32 summation bound.
"""
import numpy as np
import pytest
import torch

import oracle
import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import bf16_to_f64, dev, fp32_sum_bound, require_gpu, say
from tests.layout_ref import to_row_major

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32
CHUNK = 1 << 15  # rows compared per device step


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _periodic(block_d: torch.Tensor, n: int) -> torch.Tensor:
    """n rows, row i = block row i mod P (on the device)."""
    idx = torch.arange(n, device=block_d.device) % block_d.shape[0]
    return block_d.index_select(0, idx)


def _untile(values: torch.Tensor, meta: torch.Tensor, M: int, K: int, esize: int):
    """Row-major views (Mp x Kp/2 values as bytes, Mp x Kp/8 metadata) of the tiled compressed buffers, on the
    device: a tile is 16 rows x 64 bytes of values (KT = 128 / esize dense columns) and 16 rows x KT/8 bytes of
    metadata, tiles row block by row block and along K inside one, each tile's rows cut in four quarters
    stored quarter-major."""
    kt = 128 // esize
    Mp, Kp = (M + 15) // 16 * 16, (K + kt - 1) // kt * kt
    tiles = Kp // kt
    vb = values.view(torch.uint8).view(Mp // 16, tiles, 4, 16, 16).permute(0, 3, 1, 2, 4).reshape(Mp, tiles * 64)
    q = kt // 32
    mb = meta.view(Mp // 16, tiles, 4, 16, q).permute(0, 3, 1, 2, 4).reshape(Mp, tiles * 4 * q)
    return vb, mb


def _rows_equal_periodic(got: torch.Tensor, block_d: torch.Tensor) -> bool:
    """got[i] == block[i mod P] for every row, bit for bit (compared as bytes), chunk by chunk."""
    P = block_d.shape[0]
    got = got.reshape(-1).view(got.shape)  # unit strides (a transposed single-token output has another)
    g8 = got.view(torch.uint8) if got.dtype != torch.uint8 else got
    b8 = block_d.view(torch.uint8) if block_d.dtype != torch.uint8 else block_d
    for i0 in range(0, got.shape[0], CHUNK):
        i1 = min(i0 + CHUNK, got.shape[0])
        idx = torch.arange(i0, i1, device=got.device) % P
        if not torch.equal(g8[i0:i1], b8.index_select(0, idx)):
            return False
    return True


def _within_periodic(got: torch.Tensor, ref_d: torch.Tensor, bound_d: torch.Tensor) -> float:
    """Largest |got[i] - ref[i mod P]| / bound[i mod P] over all rows (float64 on the device)."""
    P = ref_d.shape[0]
    worst = 0.0
    for i0 in range(0, got.shape[0], CHUNK):
        i1 = min(i0 + CHUNK, got.shape[0])
        idx = torch.arange(i0, i1, device=got.device) % P
        d = (got[i0:i1].double() - ref_d.index_select(0, idx)).abs() / bound_d.index_select(0, idx)
        worst = max(worst, float(d.max()))
    return worst


@pytest.mark.parametrize("dt", ["bf16", "i8"])
def test_weight_beyond_4gib(dt):
    """An 8.6 GB weight whose compressed values take 4.3 GB: prune/compress, decompress and the GEMMs at 1, 16
    and 80 tokens (the few-token, skinny and tiled kernels) over every one of its rows."""
    esize = 2 if dt == "bf16" else 1
    K = 16384 if dt == "bf16" else 32768
    P, M = 997, 262184  # M: 16386 row blocks and 8 rows (ragged)
    odt = oracle.BF16 if dt == "bf16" else oracle.I8
    if dt == "bf16":
        Wb = synth.normal_bf16(71, (P, K), 0.02)
        Wb_d = dev(Wb, "bf16")
    else:
        Wb = np.random.default_rng(72).integers(-128, 128, size=(P, K), dtype=np.int8)
        Wb_d = dev(Wb)
    # the 2^32-byte wraps of the weight and of the values buffer, in rows, are not multiples of P
    assert (GIB4 // (K * esize)) % P != 0 and (GIB4 // (K // 2 * esize)) % P != 0
    say(f"beyond 4 GiB: {dt} weight {M} x {K} ({M * K * esize / 2**30:.1f} GiB): prune/compress")
    W_d = _periodic(Wb_d, M)
    v, m = sp.sp24_prune_compress(W_d)
    assert v.numel() * esize > GIB4
    rv, rm = oracle.prune_compress(Wb, odt)
    ref_v, ref_m = to_row_major(rv, rm, P, K, esize)
    gv, gm = _untile(v, m, M, K, esize)
    torch.cuda.synchronize()
    assert _rows_equal_periodic(gv[:M], dev(np.ascontiguousarray(ref_v).view(np.uint8)))
    assert _rows_equal_periodic(gm[:M], dev(np.ascontiguousarray(ref_m)))
    # padded rows: value 0, metadata nibbles 0x4 (positions 0 and 1)
    assert bool((gv[M:] == 0).all()) and bool((gm[M:] == 0x44).all())
    del gv, gm

    say(f"beyond 4 GiB: {dt} weight {M} x {K}: decompress")
    D_d = sp.sp24_decompress(v, m, M, K)
    Db = oracle.decompress(rv, rm, odt, P, K)
    assert _rows_equal_periodic(D_d, dev(Db, "bf16") if dt == "bf16" else dev(Db))
    del D_d, W_d
    torch.cuda.empty_cache()

    rng = np.random.default_rng(73)
    scale = (rng.random(P) * 1e-3 + 1e-4).astype(np.float32)
    scale_d = _periodic(dev(scale).view(P, 1), M).view(M)
    for N, layout in ((1, "token"), (16, "token"), (80, "token"), (80, "feature")):
        say(f"beyond 4 GiB: {dt} weight {M} x {K}: GEMM N = {N}, {layout}-major")
        if dt == "bf16":
            X = synth.normal_bf16(74 + N, (K, N))
            Xd = dev(X if layout == "feature" else np.ascontiguousarray(X.T), "bf16")
            Y = sp.sp24_gemm_bf16_ex(v, m, M, Xd, layout=layout, out_dtype=torch.float32)
            Yb = oracle.gemm_bf16(rv, rm, X, P)  # P x N, fp64
            bound = fp32_sum_bound(np.abs(bf16_to_f64(Db)) @ np.abs(bf16_to_f64(X)), K)
            Ym = Y if layout == "feature" else Y.t()
            worst = _within_periodic(Ym, dev(Yb), dev(bound))
            assert worst <= 1.0, (N, layout, worst)
        else:
            X = rng.integers(-128, 128, size=(K, N), dtype=np.int8)
            Xd = dev(X if layout == "feature" else np.ascontiguousarray(X.T))
            Yacc = sp.sp24_gemm_i8_ex(v, m, M, Xd, layout=layout)
            Ys = sp.sp24_gemm_i8_ex(v, m, M, Xd, scale=scale_d, layout=layout)
            acc, Yf = oracle.gemm_i8(rv, rm, X, P, scale)
            pick = (lambda Y: Y) if layout == "feature" else (lambda Y: Y.t().contiguous())
            assert _rows_equal_periodic(pick(Yacc), dev(acc.astype(np.int32))), (N, layout)
            assert _rows_equal_periodic(pick(Ys), dev(Yf)), (N, layout)
        del Xd
    torch.cuda.empty_cache()


# (M, K, N): activations of 4.9 GB with a 634 MB output; a 307 MB input with a 4.9 GB output
BF16_SHAPES = [(264, 4096, 600000), (4096, 256, 300000)]


@pytest.mark.parametrize("M,K,N", BF16_SHAPES)
def test_bf16_activations_or_output_beyond_4gib(M, K, N):
    """Token n of X is token n mod P of a seeded block: both layouts of the tiled kernel, every output
    element against the oracle's block product within the fp32 summation bound."""
    P = 4093
    W = synth.normal_bf16(81, (M, K), 0.02)
    Xb = synth.normal_bf16(82, (P, K))  # token-major block
    say(f"beyond 4 GiB: bf16 activations {N} x {K}, output {N} x {M}")
    v, m = sp.sp24_prune_compress(dev(W, "bf16"))
    rv, rm = oracle.prune_compress(W, oracle.BF16)
    D = bf16_to_f64(oracle.decompress(rv, rm, oracle.BF16, M, K))
    Yb = oracle.gemm_bf16(rv, rm, Xb, M, layout="token")  # P x M
    bound = fp32_sum_bound(np.abs(bf16_to_f64(Xb)) @ np.abs(D).T, K)
    Yb_d, bound_d = dev(Yb), dev(bound)
    Xb_d = dev(Xb, "bf16")
    for layout in ("token", "feature"):
        say(f"beyond 4 GiB: bf16 {M} x {K} x {N}, {layout}-major")
        if layout == "token":
            Xd = _periodic(Xb_d, N)
            assert (GIB4 // (K * 2)) % P != 0
        else:
            Xd = _periodic(Xb_d, N).t().contiguous()  # K x N
        Y = sp.sp24_gemm_bf16_ex(v, m, M, Xd, layout=layout, out_dtype=torch.float32)
        assert max(Xd.numel() * 2, Y.numel() * 4) > GIB4
        del Xd
        Yt = Y if layout == "token" else Y.t()
        worst = _within_periodic(Yt, Yb_d, bound_d)
        assert worst <= 1.0, (layout, worst)
        del Y, Yt
        torch.cuda.empty_cache()


def test_int8_activations_beyond_4gib():
    """int8 X of 4.9 GB (600000 tokens x 8192 channels) in both layouts, fp32 dequantized output bit-exact."""
    M, K, N, P = 264, 8192, 600000, 4093
    rng = np.random.default_rng(91)
    W = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    Xb = rng.integers(-128, 128, size=(P, K), dtype=np.int8)
    scale = (rng.random(M) * 1e-3 + 1e-4).astype(np.float32)
    say(f"beyond 4 GiB: int8 activations {N} x {K}")
    v, m = sp.sp24_prune_compress(dev(W))
    rv, rm = oracle.prune_compress(W, oracle.I8)
    _, Yb = oracle.gemm_i8(rv, rm, Xb, M, scale, layout="token")  # P x M
    Yb_d, Xb_d, scale_d = dev(np.ascontiguousarray(Yb)), dev(Xb), dev(scale)
    assert (GIB4 // K) % P != 0
    for layout in ("token", "feature"):
        say(f"beyond 4 GiB: int8 {M} x {K} x {N}, {layout}-major")
        Xd = _periodic(Xb_d, N) if layout == "token" else _periodic(Xb_d, N).t().contiguous()
        assert Xd.numel() > GIB4
        Y = sp.sp24_gemm_i8_ex(v, m, M, Xd, scale=scale_d, layout=layout)
        del Xd
        Yt = Y if layout == "token" else Y.t().contiguous()
        assert _rows_equal_periodic(Yt, Yb_d), layout
        del Y, Yt
        torch.cuda.empty_cache()
