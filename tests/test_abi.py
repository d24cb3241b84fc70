"""Host-side checks of the C-ABI library (no GPU needed, no kernel launched):
the library loads, exports every symbol include/*.h declares, and rejects invalid arguments on
the host before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

import structured_sparse_gemm_sp24_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    inc = os.path.join(ROOT, "include")
    txt = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sp24_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sp.LIB_PATH):
        from structured_sparse_gemm_sp24_amd import build
        build.build()
    return sp.load_library()


def test_every_declared_symbol_is_exported(lib):
    decl = _declared_functions()
    assert set(decl) == set(sp.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert sp.status_string(st) and "unknown" not in sp.status_string(st)
    assert "unknown" in sp.status_string(12345)


# Fake 16-byte-aligned addresses: every call below must be rejected before anything touches them.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10008)  # 8-byte aligned only
NULL = None


@pytest.mark.parametrize("args,expect", [
    ((NULL, 16, 8, 8, A, NULL), sp.SP24_ERR_NULL),
    ((A, 16, 8, 8, NULL, NULL), sp.SP24_ERR_NULL),
    ((A, 0, 8, 8, B, NULL), sp.SP24_ERR_SHAPE),
    ((A, 16, 0, 8, B, NULL), sp.SP24_ERR_SHAPE),
    ((A, 16, 8, 7, B, NULL), sp.SP24_ERR_SHAPE),
    ((MIS, 16, 8, 8, B, NULL), sp.SP24_ERR_ALIGN),
])
def test_col_norms_validation(lib, args, expect):
    assert lib.sp24_col_norms(*args) == expect


BF16, FP16, FP32, I8, I32 = sp.SP24_BF16, sp.SP24_FP16, sp.SP24_FP32, sp.SP24_I8, sp.SP24_I32
MAG, WANDA = sp.SP24_SCORE_MAGNITUDE, sp.SP24_SCORE_WANDA


@pytest.mark.parametrize("args,expect", [
    # W, dtype, M, K, ldw, score, norms, values, val_dtype, meta, stream
    ((NULL, BF16, 4, 16, 16, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_NULL),
    ((A, BF16, 4, 16, 16, MAG, NULL, NULL, BF16, C, NULL), sp.SP24_ERR_NULL),
    ((A, BF16, 4, 16, 16, MAG, NULL, B, BF16, NULL, NULL), sp.SP24_ERR_NULL),
    ((A, I32, 4, 16, 16, MAG, NULL, B, I32, C, NULL), sp.SP24_ERR_DTYPE),
    ((A, BF16, 4, 16, 16, MAG, NULL, B, FP32, C, NULL), sp.SP24_ERR_DTYPE),
    ((A, FP16, 4, 16, 16, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_DTYPE),
    ((A, I8, 4, 16, 16, WANDA, A, B, I8, C, NULL), sp.SP24_ERR_DTYPE),
    ((A, BF16, 4, 16, 16, WANDA, NULL, B, BF16, C, NULL), sp.SP24_ERR_NULL),
    ((A, BF16, 4, 16, 16, MAG, A, B, BF16, C, NULL), sp.SP24_ERR_ARG),
    ((A, BF16, 4, 16, 16, 7, NULL, B, BF16, C, NULL), sp.SP24_ERR_ARG),
    ((A, BF16, 0, 16, 16, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_SHAPE),
    ((A, BF16, 4, 8, 8, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_SHAPE),
    ((A, BF16, 4, 24, 24, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_SHAPE),
    ((A, BF16, 4, 32, 16, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_SHAPE),
    ((A, BF16, 4, 16, 20, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_ALIGN),  # 40-byte rows
    ((MIS, BF16, 4, 16, 16, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_ALIGN),
    ((A, FP32, 4, 16, 16, WANDA, MIS, B, BF16, C, NULL), sp.SP24_ERR_ALIGN),
    ((A, I8, 4, 16, 24, MAG, NULL, B, I8, C, NULL), sp.SP24_ERR_ALIGN),
    # rows x chunks per row past 2^63 (the check must not overflow into a small product)
    ((A, BF16, 1 << 61, 1 << 20, 1 << 20, MAG, NULL, B, BF16, C, NULL), sp.SP24_ERR_SHAPE),
])
def test_prune_compress_validation(lib, args, expect):
    assert lib.sp24_prune_compress(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((NULL, B, BF16, 4, 16, C, 16, NULL), sp.SP24_ERR_NULL),
    ((A, B, I32, 4, 16, C, 16, NULL), sp.SP24_ERR_DTYPE),
    ((A, B, BF16, 4, 40, C, 40, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, BF16, 4, 16, C, 8, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, FP32, 4, 16, C, 18, NULL), sp.SP24_ERR_ALIGN),
    ((A, MIS, BF16, 4, 16, C, 16, NULL), sp.SP24_ERR_ALIGN),
    # one thread per 16-column chunk of the padded tiles must fit 32 bits: 2^20 x 2^16 is 2^32 chunks, and
    # 2^20 - 1 rows pad to 2^20 (the unpadded count alone would pass)
    ((A, B, BF16, 1 << 20, 1 << 16, C, 1 << 16, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, BF16, (1 << 20) - 1, 1 << 16, C, 1 << 16, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, BF16, 1 << 61, 1 << 20, C, 1 << 20, NULL), sp.SP24_ERR_SHAPE),  # product past 2^63
])
def test_decompress_validation(lib, args, expect):
    assert lib.sp24_decompress(*args) == expect


@pytest.mark.parametrize("args,expect", [
    # values, meta, M, K, X, N, ldx, Y, out_dtype, ldy, stream
    ((NULL, B, 16, 16, C, 4, 4, A, FP32, 4, NULL), sp.SP24_ERR_NULL),
    ((A, B, 16, 16, C, 4, 4, NULL, FP32, 4, NULL), sp.SP24_ERR_NULL),
    ((A, B, 16, 16, C, 4, 4, A, I8, 4, NULL), sp.SP24_ERR_DTYPE),
    ((A, B, 0, 16, C, 4, 4, A, FP32, 4, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 0, 4, A, FP32, 4, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 20, C, 4, 4, A, FP32, 4, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 4, 3, A, FP32, 4, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 4, 4, A, FP32, 3, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, MIS, 4, 4, A, FP32, 4, NULL), sp.SP24_ERR_ALIGN),
])
def test_gemm_bf16_validation(lib, args, expect):
    assert lib.sp24_gemm_bf16(*args) == expect


@pytest.mark.parametrize("args,expect", [
    # values, meta, M, K, X, N, ldx, scale, Y, ldy, stream
    ((NULL, B, 16, 16, C, 4, 4, NULL, A, 4, NULL), sp.SP24_ERR_NULL),
    ((A, B, 16, 262144, C, 4, 4, NULL, A, 4, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 4, 4, ctypes.c_void_p(0x10002), A, 4, NULL), sp.SP24_ERR_ALIGN),
    ((A, B, 16, 16, C, 5, 4, NULL, A, 5, NULL), sp.SP24_ERR_SHAPE),
])
def test_gemm_i8_validation(lib, args, expect):
    assert lib.sp24_gemm_i8(*args) == expect


FM, TM = sp.SP24_FEATURE_MAJOR, sp.SP24_TOKEN_MAJOR


@pytest.mark.parametrize("args,expect", [
    # values, meta, M, K, X, N, ldx, x_batch_stride, Y, out_dtype, ldy, y_batch_stride, batch, layout, stream
    ((A, B, 16, 16, C, 4, 4, 0, A, FP32, 4, 0, 1, 2, NULL), sp.SP24_ERR_ARG),      # unknown layout
    ((A, B, 16, 16, C, 4, 4, 0, A, FP32, 4, 0, 0, FM, NULL), sp.SP24_ERR_SHAPE),   # batch 0
    ((A, B, 16, 16, C, 4, 8, 0, A, FP32, 16, 0, 1, TM, NULL), sp.SP24_ERR_SHAPE),  # token-major ldx < K
    ((A, B, 16, 16, C, 4, 16, 0, A, FP32, 8, 0, 1, TM, NULL), sp.SP24_ERR_SHAPE),  # token-major ldy < M
    ((A, B, 16, 16, C, 4, 4, 64, A, FP32, 4, 32, 2, FM, NULL), sp.SP24_ERR_SHAPE),  # Y entries overlap
    ((A, B, 16, 16, C, 4, 4, 64, A, FP32, 4, -64, 2, FM, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 4, 4, -8, A, FP32, 4, 64, 2, FM, NULL), sp.SP24_ERR_SHAPE),  # negative X stride
    ((A, B, 16, 16, C, 4, 4, 4, A, FP32, 4, 64, 2, FM, NULL), sp.SP24_ERR_ALIGN),   # X entry 8 bytes apart
    ((A, B, 16, 16, C, 4, 4, 64, A, FP32, 4, 66, 2, FM, NULL), sp.SP24_ERR_ALIGN),  # Y entry misaligned
    ((A, B, 16, 16, C, 4, 4, 0, A, I32, 4, 0, 1, FM, NULL), sp.SP24_ERR_DTYPE),
    ((NULL, B, 16, 16, C, 4, 4, 0, A, FP32, 4, 0, 1, TM, NULL), sp.SP24_ERR_NULL),
])
def test_gemm_bf16_ex_validation(lib, args, expect):
    assert lib.sp24_gemm_bf16_ex(*args) == expect


@pytest.mark.parametrize("args,expect", [
    # values, meta, M, K, X, N, ldx, x_batch_stride, scale, Y, ldy, y_batch_stride, batch, layout, stream
    ((A, B, 16, 16, C, 4, 16, 0, NULL, A, 16, 0, 1, 7, NULL), sp.SP24_ERR_ARG),
    ((A, B, 16, 16, C, 4, 8, 0, NULL, A, 16, 0, 1, TM, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 4, 16, 0, NULL, A, 4, 0, 1, TM, NULL), sp.SP24_ERR_SHAPE),
    ((A, B, 16, 16, C, 4, 4, 8, NULL, A, 4, 64, 2, FM, NULL), sp.SP24_ERR_ALIGN),
    ((A, B, 16, 262144, C, 4, 262144, 0, NULL, A, 16, 0, 1, TM, NULL), sp.SP24_ERR_SHAPE),
])
def test_gemm_i8_ex_validation(lib, args, expect):
    assert lib.sp24_gemm_i8_ex(*args) == expect


@pytest.mark.parametrize("args,expect", [
    # values, meta, M, K, X, N, ldx, xbs, scale, bias, act, Y, out_dtype, out_scale, ldy, ybs, batch, layout, stream
    ((A, B, 16, 16, C, 4, 4, 0, NULL, NULL, 0, A, FP32, 1.0, 4, 0, 1, FM, NULL), sp.SP24_ERR_NULL),    # no scale
    ((A, B, 16, 16, C, 4, 4, 0, B, NULL, 0, A, I32, 1.0, 4, 0, 1, FM, NULL), sp.SP24_ERR_DTYPE),
    ((A, B, 16, 16, C, 4, 4, 0, B, NULL, 2, A, FP32, 1.0, 4, 0, 1, FM, NULL), sp.SP24_ERR_ARG),       # activation
    ((A, B, 16, 16, C, 4, 4, 0, B, NULL, 1, A, I8, 0.0, 4, 0, 1, FM, NULL), sp.SP24_ERR_ARG),         # out_scale
    ((A, B, 16, 16, C, 4, 4, 0, B, NULL, 1, A, I8, float("nan"), 4, 0, 1, FM, NULL), sp.SP24_ERR_ARG),
    ((A, B, 16, 16, C, 4, 4, 0, B, ctypes.c_void_p(0x20002), 0, A, FP32, 1.0, 4, 0, 1, FM, NULL), sp.SP24_ERR_ALIGN),
    ((A, B, 16, 16, C, 4, 4, 8, B, NULL, 0, A, I8, 1.0, 4, 64, 2, FM, NULL), sp.SP24_ERR_ALIGN),      # X stride
    ((A, B, 16, 16, C, 4, 16, 0, B, NULL, 0, A, BF16, 1.0, 8, 0, 1, TM, NULL), sp.SP24_ERR_SHAPE),    # ldy < M
])
def test_gemm_i8_fused_validation(lib, args, expect):
    assert lib.sp24_gemm_i8_fused(*args) == expect


@pytest.mark.parametrize("args,expect", [
    # W, dtype, M, K, ldw, keep, score, norms, mask, W_out, ldo, stream
    ((NULL, BF16, 16, 16, 16, 2, 0, NULL, B, NULL, 16, NULL), sp.SP24_ERR_NULL),
    ((A, BF16, 16, 16, 16, 2, 0, NULL, NULL, NULL, 16, NULL), sp.SP24_ERR_NULL),   # neither output
    ((A, BF16, 16, 16, 16, 0, 0, NULL, B, NULL, 16, NULL), sp.SP24_ERR_ARG),       # keep 0
    ((A, BF16, 16, 16, 16, 5, 0, NULL, B, NULL, 16, NULL), sp.SP24_ERR_ARG),       # keep 5
    ((A, I32, 16, 16, 16, 2, 0, NULL, B, NULL, 16, NULL), sp.SP24_ERR_DTYPE),
    ((A, I8, 16, 16, 16, 2, 1, C, B, NULL, 16, NULL), sp.SP24_ERR_DTYPE),          # Wanda on int8
    ((A, BF16, 16, 16, 16, 2, 0, C, B, NULL, 16, NULL), sp.SP24_ERR_ARG),          # norms with magnitude
    ((A, BF16, 16, 20, 24, 2, 0, NULL, B, NULL, 24, NULL), sp.SP24_ERR_SHAPE),     # K % 16
    ((A, BF16, 16, 16, 16, 2, 0, NULL, NULL, C, 8, NULL), sp.SP24_ERR_SHAPE),      # ldo < K
    ((A, BF16, 16, 16, 16, 2, 0, NULL, MIS, NULL, 16, NULL), sp.SP24_ERR_ALIGN),
    ((A, BF16, 16, 16, 20, 2, 0, NULL, B, NULL, 16, NULL), sp.SP24_ERR_ALIGN),     # ldw*2 % 16
    ((A, BF16, 1 << 61, 1 << 20, 1 << 20, 2, 0, NULL, B, NULL, 1 << 20, NULL), sp.SP24_ERR_SHAPE),  # past 2^63
])
def test_prune_mask_validation(lib, args, expect):
    assert lib.sp24_prune_mask(*args) == expect


@pytest.mark.parametrize("args,expect", [
    # W, dtype, M, K, ldw, score, norms, sweeps, perm, stream
    ((NULL, BF16, 16, 16, 16, 0, NULL, 1, B, NULL), sp.SP24_ERR_NULL),
    ((A, BF16, 16, 16, 16, 0, NULL, 1, NULL, NULL), sp.SP24_ERR_NULL),
    ((A, I32, 16, 16, 16, 0, NULL, 1, B, NULL), sp.SP24_ERR_DTYPE),
    ((A, BF16, 16, 16, 16, 0, NULL, -1, B, NULL), sp.SP24_ERR_ARG),
    ((A, BF16, 16, 16, 16, 0, C, 1, B, NULL), sp.SP24_ERR_ARG),        # norms with magnitude
    ((A, I8, 16, 16, 16, 1, C, 1, B, NULL), sp.SP24_ERR_DTYPE),        # Wanda on int8
    ((A, BF16, 16, 6, 16, 0, NULL, 1, B, NULL), sp.SP24_ERR_SHAPE),    # K % 4
    ((A, BF16, 16, 4, 16, 0, NULL, 1, B, NULL), sp.SP24_ERR_SHAPE),    # K < 8
    ((A, BF16, 16, 16, 8, 0, NULL, 1, B, NULL), sp.SP24_ERR_SHAPE),    # ldw < K
    ((A, BF16, 16, 16, 16, 0, NULL, 1, ctypes.c_void_p(0x20002), NULL), sp.SP24_ERR_ALIGN),
])
def test_channel_permutation_validation(lib, args, expect):
    assert lib.sp24_channel_permutation(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((4, 10, NULL, NULL), sp.SP24_ERR_NULL),
    ((0, 10, A, NULL), sp.SP24_ERR_ARG),
    ((65536, 10, A, NULL), sp.SP24_ERR_ARG),
    ((4, 0, A, NULL), sp.SP24_ERR_ARG),
    ((4, 1000001, A, NULL), sp.SP24_ERR_ARG),
    ((4, 10, ctypes.c_void_p(0x10004), NULL), sp.SP24_ERR_ALIGN),
])
def test_probe_sclk_validation(lib, args, expect):
    assert lib.sp24_probe_sclk(*args) == expect


def test_compressed_bytes(lib):
    vb, mb = ctypes.c_int64(), ctypes.c_int64()
    # rows padded to 16, columns to 128 / value size
    for M, K, dt, want in [(3072, 768, BF16, (3072 * 384 * 2, 3072 * 96)), (1, 16, BF16, (16 * 32 * 2, 16 * 8)),
                           (17, 48, I8, (32 * 64, 32 * 16)), (5, 16, FP32, (16 * 16 * 4, 16 * 4))]:
        assert lib.sp24_compressed_bytes(M, K, dt, ctypes.byref(vb), ctypes.byref(mb)) == sp.SP24_OK
        assert (vb.value, mb.value) == want
    assert lib.sp24_compressed_bytes(4, 20, BF16, ctypes.byref(vb), ctypes.byref(mb)) == sp.SP24_ERR_SHAPE
    assert lib.sp24_compressed_bytes(4, 16, I32, ctypes.byref(vb), ctypes.byref(mb)) == sp.SP24_ERR_DTYPE
    assert lib.sp24_compressed_bytes(4, 16, BF16, None, ctypes.byref(mb)) == sp.SP24_ERR_NULL


def test_compressed_bytes_matches_oracle(lib):
    import oracle
    for M, K in [(1, 16), (37, 208), (3072, 768)]:
        for dt in (BF16, FP32, I8):
            assert sp.sp24_compressed_bytes(M, K, {BF16: torch.bfloat16, FP32: torch.float32, I8: torch.int8}[dt]) == \
                oracle.compressed_bytes(M, K, dt)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="only meaningful where no GPU is visible")
def test_valid_arguments_without_a_device_report_device_error(lib):
    # all host checks pass, then the device check fails: nothing is launched
    assert lib.sp24_gemm_bf16(A, B, 16, 16, C, 4, 4, A, FP32, 4, NULL) == sp.SP24_ERR_DEVICE
    assert lib.sp24_gemm_bf16_ex(A, B, 16, 16, C, 4, 16, 64, A, FP32, 16, 64, 2, TM, NULL) == sp.SP24_ERR_DEVICE
    assert lib.sp24_gemm_i8_ex(A, B, 16, 16, C, 4, 16, 64, NULL, A, 16, 64, 2, TM, NULL) == sp.SP24_ERR_DEVICE
    assert lib.sp24_gemm_i8_fused(A, B, 16, 16, C, 4, 16, 64, B, NULL, 1, A, I8, 0.5, 16, 64, 2, TM, NULL) == \
        sp.SP24_ERR_DEVICE
    assert lib.sp24_col_norms(A, 16, 8, 8, B, NULL) == sp.SP24_ERR_DEVICE


def test_binding_refuses_host_tensors(lib):
    with pytest.raises(ValueError):
        sp.sp24_col_norms(torch.zeros((4, 4), dtype=torch.bfloat16))


def test_bench_dense_reference_validation(lib):
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    b = I64()
    assert lib.sp24_bench_dense_tiled_bytes(40, 128, ctypes.byref(b)) == 0 and b.value == 48 * 128 * 2
    assert lib.sp24_bench_dense_tiled_bytes(40, 96, ctypes.byref(b)) == sp.SP24_ERR_SHAPE
    assert lib.sp24_bench_dense_tiled_bytes(40, 128, None) == sp.SP24_ERR_NULL
    p = P(4096)
    assert lib.sp24_bench_dense_tile(None, 16, 64, 64, p, None) == sp.SP24_ERR_NULL
    assert lib.sp24_bench_dense_tile(p, 16, 96, 96, p, None) == sp.SP24_ERR_SHAPE
    assert lib.sp24_bench_dense_tile(p, 16, 64, 60, p, None) == sp.SP24_ERR_SHAPE
    assert lib.sp24_bench_dense_tile(p, 16, 64, 68, p, None) == sp.SP24_ERR_ALIGN
    assert lib.sp24_bench_dense_tile(P(4098), 16, 64, 64, p, None) == sp.SP24_ERR_ALIGN
    g = lib.sp24_bench_gemm_dense_bf16
    assert g(p, 16, 64, None, 8, 64, p, sp.SP24_FP32, 16, None) == sp.SP24_ERR_NULL
    assert g(p, 16, 64, p, 8, 64, p, sp.SP24_I8, 16, None) == sp.SP24_ERR_DTYPE
    assert g(p, 16, 80, p, 8, 80, p, sp.SP24_FP32, 16, None) == sp.SP24_ERR_SHAPE
    assert g(p, 16, 64, p, 0, 64, p, sp.SP24_FP32, 16, None) == sp.SP24_ERR_SHAPE
    assert g(p, 16, 64, p, 8, 64, p, sp.SP24_FP32, 15, None) == sp.SP24_ERR_SHAPE
    assert g(p, 16, 64, p, 8, 68, p, sp.SP24_FP32, 16, None) == sp.SP24_ERR_ALIGN


def test_bench_stream_read_validation(lib):
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    b = I64()
    assert lib.sp24_bench_stream_read_blocks(100, ctypes.byref(b)) == sp.SP24_ERR_SHAPE
    assert lib.sp24_bench_stream_read_blocks(64, None) == sp.SP24_ERR_NULL
    assert lib.sp24_bench_stream_read(None, 64, P(4096), None) == sp.SP24_ERR_NULL
    assert lib.sp24_bench_stream_read(P(4096), 8, P(4096), None) == sp.SP24_ERR_SHAPE
    assert lib.sp24_bench_stream_read(P(4104), 64, P(4096), None) == sp.SP24_ERR_ALIGN
