"""sp24: 2:4 structured-sparse prune/compress and sparse GEMM for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libsp24.so`` (declared in include/sp24.h): the functions
below have the C entry points' names and only marshal arguments -- torch tensors supply device
memory and the current HIP stream; every step runs in the library's HIP kernels. If the library is
not built, or the device is not gfx950, the calls raise; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsp24.so")

SP24_OK, SP24_ERR_NULL, SP24_ERR_SHAPE, SP24_ERR_ALIGN = 0, -1, -2, -3
SP24_ERR_DTYPE, SP24_ERR_ARG, SP24_ERR_DEVICE, SP24_ERR_HIP = -4, -5, -6, -7
SP24_BF16, SP24_FP16, SP24_FP32, SP24_I8, SP24_I32 = 0, 1, 2, 3, 4
SP24_SCORE_MAGNITUDE, SP24_SCORE_WANDA = 0, 1
SP24_FEATURE_MAJOR, SP24_TOKEN_MAJOR = 0, 1
SP24_ACT_NONE, SP24_ACT_GELU = 0, 1

# every symbol include/sp24.h declares
EXPORTS = ("sp24_col_norms", "sp24_compressed_bytes", "sp24_prune_compress", "sp24_prune_mask",
           "sp24_channel_permutation", "sp24_decompress",
           "sp24_gemm_bf16",
           "sp24_gemm_i8", "sp24_gemm_bf16_ex", "sp24_gemm_i8_ex", "sp24_gemm_i8_fused", "sp24_probe_sclk",
           "sp24_bench_dense_tiled_bytes", "sp24_bench_dense_tile", "sp24_bench_gemm_dense_bf16",
           "sp24_bench_stream_read_blocks", "sp24_bench_stream_read",
           "sp24_status_string")

_TORCH_TO_SP24 = {torch.bfloat16: SP24_BF16, torch.float16: SP24_FP16, torch.float32: SP24_FP32,
                  torch.int8: SP24_I8, torch.int32: SP24_I32}
_SP24_TO_TORCH = {v: k for k, v in _TORCH_TO_SP24.items()}


class Sp24Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsp24.so (built by ``structured_sparse_gemm_sp24_amd.build``). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m structured_sparse_gemm_sp24_amd.build` "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.sp24_col_norms.argtypes = [P, I64, I64, I64, P, P]
    lib.sp24_compressed_bytes.argtypes = [I64, I64, I, ctypes.POINTER(I64), ctypes.POINTER(I64)]
    lib.sp24_prune_compress.argtypes = [P, I, I64, I64, I64, I, P, P, I, P, P]
    lib.sp24_decompress.argtypes = [P, P, I, I64, I64, P, I64, P]
    lib.sp24_prune_mask.argtypes = [P, I, I64, I64, I64, I, I, P, P, P, I64, P]
    lib.sp24_channel_permutation.argtypes = [P, I, I64, I64, I64, I, P, I, P, P]
    lib.sp24_gemm_bf16.argtypes = [P, P, I64, I64, P, I64, I64, P, I, I64, P]
    lib.sp24_gemm_i8.argtypes = [P, P, I64, I64, P, I64, I64, P, P, I64, P]
    lib.sp24_gemm_bf16_ex.argtypes = [P, P, I64, I64, P, I64, I64, I64, P, I, I64, I64, I64, I, P]
    lib.sp24_gemm_i8_ex.argtypes = [P, P, I64, I64, P, I64, I64, I64, P, P, I64, I64, I64, I, P]
    lib.sp24_gemm_i8_fused.argtypes = [P, P, I64, I64, P, I64, I64, I64, P, P, I, P, I, ctypes.c_float, I64, I64, I64,
                                       I, P]
    lib.sp24_probe_sclk.argtypes = [I64, I, P, P]
    lib.sp24_bench_dense_tiled_bytes.argtypes = [I64, I64, ctypes.POINTER(I64)]
    lib.sp24_bench_dense_tile.argtypes = [P, I64, I64, I64, P, P]
    lib.sp24_bench_gemm_dense_bf16.argtypes = [P, I64, I64, P, I64, I64, P, I, I64, P]
    lib.sp24_bench_stream_read_blocks.argtypes = [I64, ctypes.POINTER(I64)]
    lib.sp24_bench_stream_read.argtypes = [P, I64, P, P]
    for fn in EXPORTS[:-1]:
        getattr(lib, fn).restype = I
    lib.sp24_status_string.argtypes = [I]
    lib.sp24_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().sp24_status_string(int(status)).decode()


def _check(fn: str, st: int):
    if st != SP24_OK:
        raise Sp24Error(fn, st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _rows(t: torch.Tensor, name: str) -> int:
    """Row pitch of a 2-D tensor with unit column stride."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _dev_check(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("sp24 operates on device tensors only")


def sp24_col_norms(X: torch.Tensor, norms: torch.Tensor | None = None) -> torch.Tensor:
    """norms[j] = ||X[j, :]||_2 for bf16 X (K x N, row pitch = X.stride(0)); returns fp32[K]."""
    _dev_check(X)
    K, N = X.shape
    if norms is None:
        norms = torch.empty(K, dtype=torch.float32, device=X.device)
    _check("sp24_col_norms", load_library().sp24_col_norms(_ptr(X), K, N, _rows(X, "X"), _ptr(norms), _stream(X)))
    return norms


_ESIZE = {torch.bfloat16: 2, torch.float16: 2, torch.float32: 4, torch.int8: 1}


def sp24_compressed_bytes(M: int, K: int, val_dtype: torch.dtype):
    """(values bytes, metadata bytes) of the compressed form of an M x K weight."""
    vb, mb = ctypes.c_int64(), ctypes.c_int64()
    _check("sp24_compressed_bytes", load_library().sp24_compressed_bytes(M, K, _TORCH_TO_SP24[val_dtype],
                                                                           ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def _check_compressed(values: torch.Tensor, meta: torch.Tensor, M: int, K: int):
    vb, mb = sp24_compressed_bytes(M, K, values.dtype)
    if values.numel() * _ESIZE[values.dtype] != vb or meta.numel() != mb or meta.dtype != torch.uint8:
        raise ValueError(f"compressed buffers hold {values.numel() * _ESIZE[values.dtype]} / {meta.numel()} bytes; "
                         f"an {M} x {K} weight needs {vb} / {mb}")
    if not (values.is_contiguous() and meta.is_contiguous()):
        raise ValueError("compressed buffers must be contiguous")


def sp24_prune_compress(W: torch.Tensor, score: int = SP24_SCORE_MAGNITUDE, norms: torch.Tensor | None = None,
                        val_dtype: torch.dtype | None = None, values: torch.Tensor | None = None,
                        meta: torch.Tensor | None = None):
    """2:4 prune + compress of W (M x K). Returns (values, meta): 1-D buffers in the tiled layout of
    include/sp24.h (values of val_dtype, meta uint8), sized by sp24_compressed_bytes."""
    _dev_check(W, norms, values, meta)
    M, K = W.shape
    vdt = W.dtype if val_dtype is None else val_dtype
    vb, mb = sp24_compressed_bytes(M, K, vdt)
    if values is None:
        values = torch.empty(vb // _ESIZE[vdt], dtype=vdt, device=W.device)
    if meta is None:
        meta = torch.empty(mb, dtype=torch.uint8, device=W.device)
    _check_compressed(values, meta, M, K)
    st = load_library().sp24_prune_compress(_ptr(W), _TORCH_TO_SP24[W.dtype], M, K, _rows(W, "W"), int(score),
                                            _ptr(norms), _ptr(values), _TORCH_TO_SP24[vdt], _ptr(meta), _stream(W))
    _check("sp24_prune_compress", st)
    return values, meta


def sp24_prune_mask(W: torch.Tensor, keep: int, score: int = SP24_SCORE_MAGNITUDE, norms: torch.Tensor | None = None,
                    mask: torch.Tensor | None = None, out: torch.Tensor | None = None, want_masked: bool = True):
    """k-of-4 mask of W (M x K): returns (mask, masked W). mask is uint8 M x K/8 (nibble of group g at
    byte g/2, bit t = position t kept); the masked weight keeps the selected elements and zeroes the
    rest (None when want_masked is False and no out is given)."""
    _dev_check(W, norms, mask, out)
    M, K = W.shape
    if mask is None:
        mask = torch.empty((M, K // 8), dtype=torch.uint8, device=W.device)
    if out is None and want_masked:
        out = torch.empty((M, K), dtype=W.dtype, device=W.device)
    if mask.dtype != torch.uint8 or tuple(mask.shape) != (M, K // 8) or not mask.is_contiguous():
        raise ValueError(f"mask must be a contiguous uint8 tensor of shape {(M, K // 8)}")
    st = load_library().sp24_prune_mask(_ptr(W), _TORCH_TO_SP24[W.dtype], M, K, _rows(W, "W"), int(keep), int(score),
                                        _ptr(norms), _ptr(mask), _ptr(out), _rows(out, "out") if out is not None else K,
                                        _stream(W))
    _check("sp24_prune_mask", st)
    return mask, out


def sp24_channel_permutation(W: torch.Tensor, sweeps: int = 1, score: int = SP24_SCORE_MAGNITUDE,
                             norms: torch.Tensor | None = None, perm: torch.Tensor | None = None) -> torch.Tensor:
    """Input-channel order (int32[K]) in which 2:4 pruning of W[:, perm] keeps at least as much score."""
    _dev_check(W, norms, perm)
    M, K = W.shape
    if perm is None:
        perm = torch.empty(K, dtype=torch.int32, device=W.device)
    st = load_library().sp24_channel_permutation(_ptr(W), _TORCH_TO_SP24[W.dtype], M, K, _rows(W, "W"), int(score),
                                                 _ptr(norms), int(sweeps), _ptr(perm), _stream(W))
    _check("sp24_channel_permutation", st)
    return perm


def sp24_decompress(values: torch.Tensor, meta: torch.Tensor, M: int, K: int,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense M x K pruned weight from (values, meta); +0 at pruned slots."""
    _dev_check(values, meta, out)
    _check_compressed(values, meta, M, K)
    if out is None:
        out = torch.empty((M, K), dtype=values.dtype, device=values.device)
    st = load_library().sp24_decompress(_ptr(values), _ptr(meta), _TORCH_TO_SP24[values.dtype], M, K, _ptr(out),
                                        _rows(out, "out"), _stream(values))
    _check("sp24_decompress", st)
    return out


def sp24_gemm_bf16(values: torch.Tensor, meta: torch.Tensor, M: int, X: torch.Tensor,
                   out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = W_2:4 . X with bf16 operands and fp32 accumulation; W is M x K (K = X rows); Y is fp32 or
    bf16 (M x N)."""
    _dev_check(values, meta, X, out)
    K, N = X.shape
    _check_compressed(values, meta, M, K)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    st = load_library().sp24_gemm_bf16(_ptr(values), _ptr(meta), M, K, _ptr(X), N, _rows(X, "X"), _ptr(out),
                                       _TORCH_TO_SP24[out.dtype], _rows(out, "out"), _stream(X))
    _check("sp24_gemm_bf16", st)
    return out


def sp24_gemm_i8(values: torch.Tensor, meta: torch.Tensor, M: int, X: torch.Tensor, scale: torch.Tensor | None = None,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 sparse GEMM: int32 accumulators, or fp32 fl32(acc) * scale[m] when ``scale`` is given."""
    _dev_check(values, meta, X, scale, out)
    K, N = X.shape
    _check_compressed(values, meta, M, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32 if scale is not None else torch.int32, device=X.device)
    st = load_library().sp24_gemm_i8(_ptr(values), _ptr(meta), M, K, _ptr(X), N, _rows(X, "X"), _ptr(scale),
                                     _ptr(out), _rows(out, "out"), _stream(X))
    _check("sp24_gemm_i8", st)
    return out


def _layout(layout) -> int:
    if layout in ("feature", SP24_FEATURE_MAJOR):
        return SP24_FEATURE_MAJOR
    if layout in ("token", SP24_TOKEN_MAJOR):
        return SP24_TOKEN_MAJOR
    raise ValueError(f"layout must be 'feature' or 'token', not {layout!r}")


def _gemm_operands(X: torch.Tensor, M: int, layout: int, out: torch.Tensor | None, out_dtype: torch.dtype):
    """(K, N, ldx, x batch stride, batch, out, ldy, y batch stride) of a 2-D or batched 3-D X."""
    if X.dim() not in (2, 3):
        raise ValueError("X must be 2-D, or 3-D for a batch")
    batch = X.shape[0] if X.dim() == 3 else 1
    X2 = X[0] if X.dim() == 3 else X
    if layout == SP24_TOKEN_MAJOR:
        N, K = X2.shape
        yshape = (N, M)
    else:
        K, N = X2.shape
        yshape = (M, N)
    if out is None:
        out = torch.empty(((batch,) if X.dim() == 3 else ()) + yshape, dtype=out_dtype, device=X.device)
    if out.dim() != X.dim() or tuple(out.shape[-2:]) != yshape or (X.dim() == 3 and out.shape[0] != batch):
        raise ValueError(f"out must have shape {((batch,) if X.dim() == 3 else ()) + yshape}")
    Y2 = out[0] if out.dim() == 3 else out
    sx = X.stride(0) if X.dim() == 3 else 0
    sy = out.stride(0) if out.dim() == 3 else 0
    return K, N, _rows(X2, "X"), sx, batch, out, _rows(Y2, "out"), sy


def sp24_gemm_bf16_ex(values: torch.Tensor, meta: torch.Tensor, M: int, X: torch.Tensor, layout="feature",
                      out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 sparse GEMM in either layout, optionally batched. layout 'feature': X is K x N, Y M x N;
    'token': X is N x K (a Linear layer's input), Y N x M. A 3-D X ([batch, ...]) runs one product per
    entry with the shared weight (e.g. a 1x1 conv over NCHW images, feature-major)."""
    _dev_check(values, meta, X, out)
    lay = _layout(layout)
    K, N, ldx, sx, batch, out, ldy, sy = _gemm_operands(X, M, lay, out, out_dtype)
    _check_compressed(values, meta, M, K)
    st = load_library().sp24_gemm_bf16_ex(_ptr(values), _ptr(meta), M, K, _ptr(X), N, ldx, sx, _ptr(out),
                                          _TORCH_TO_SP24[out.dtype], ldy, sy, batch, lay, _stream(X))
    _check("sp24_gemm_bf16_ex", st)
    return out


def sp24_gemm_i8_ex(values: torch.Tensor, meta: torch.Tensor, M: int, X: torch.Tensor, scale: torch.Tensor | None = None,
                    layout="feature", out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 sparse GEMM in either layout, optionally batched (as sp24_gemm_bf16_ex); fp32 out with
    ``scale`` (per output channel m), else int32 accumulators."""
    _dev_check(values, meta, X, scale, out)
    lay = _layout(layout)
    K, N, ldx, sx, batch, out, ldy, sy = _gemm_operands(X, M, lay, out,
                                                        torch.float32 if scale is not None else torch.int32)
    _check_compressed(values, meta, M, K)
    st = load_library().sp24_gemm_i8_ex(_ptr(values), _ptr(meta), M, K, _ptr(X), N, ldx, sx, _ptr(scale), _ptr(out),
                                        ldy, sy, batch, lay, _stream(X))
    _check("sp24_gemm_i8_ex", st)
    return out


_ACT = {"none": SP24_ACT_NONE, "gelu": SP24_ACT_GELU, SP24_ACT_NONE: SP24_ACT_NONE, SP24_ACT_GELU: SP24_ACT_GELU}


def sp24_gemm_i8_fused(values: torch.Tensor, meta: torch.Tensor, M: int, X: torch.Tensor, scale: torch.Tensor,
                       bias: torch.Tensor | None = None, activation="none", out_dtype: torch.dtype = torch.float32,
                       out_scale: float = 1.0, layout="feature", out: torch.Tensor | None = None) -> torch.Tensor:
    """int8 sparse GEMM with the FFN epilogue fused: y = fl32(fl32(acc) * scale[m]) (+ bias[m]) (GELU),
    stored as fp32, bf16, or int8 codes clamp(rne(y / out_scale), -127, 127). Layout and batching as
    sp24_gemm_i8_ex."""
    _dev_check(values, meta, X, scale, bias, out)
    if scale is None:
        raise ValueError("the fused epilogue needs the dequant scale")
    lay = _layout(layout)
    K, N, ldx, sx, batch, out, ldy, sy = _gemm_operands(X, M, lay, out, out_dtype)
    _check_compressed(values, meta, M, K)
    st = load_library().sp24_gemm_i8_fused(_ptr(values), _ptr(meta), M, K, _ptr(X), N, ldx, sx, _ptr(scale),
                                           _ptr(bias), _ACT[activation], _ptr(out), _TORCH_TO_SP24[out.dtype],
                                           float(out_scale), ldy, sy, batch, lay, _stream(X))
    _check("sp24_gemm_i8_fused", st)
    return out


def sp24_probe_sclk(blocks: int | None = None, iters: int = 4000, device: int | None = None) -> dict:
    """Sustained shader clock under matrix-core load and the issue rate of back-to-back smfmacs, from
    one probe launch (one workgroup of 4 waves per compute unit by default): per wave, shader-clock
    cycles and 100 MHz real-time ticks of iters x 16 independent v_smfmac_f32_16x16x64_bf16."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    if blocks is None:
        blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.zeros(8 * blocks, dtype=torch.int64, device=dev)
    st = load_library().sp24_probe_sclk(int(blocks), int(iters), _ptr(out), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    _check("sp24_probe_sclk", st)
    h = out.view(-1, 2).cpu().double()
    cycles, ticks = h[:, 0], h[:, 1]
    n = 16.0 * iters
    return {"sclk_mhz": float((cycles / (ticks / 100.0)).mean()), "cycles_per_smfmac": float((cycles / n).mean()),
            "waves": int(h.shape[0])}


# ----------------------------------------------------------------------------- measurement support
# (include/sp24_bench.h): a dense reference GEMM with the token-major sparse kernel's tiling.

def sp24_bench_dense_tiled_bytes(M: int, K: int) -> int:
    """Bytes of the dense tiled copy of an M x K bf16 weight."""
    b = ctypes.c_int64()
    _check("sp24_bench_dense_tiled_bytes", load_library().sp24_bench_dense_tiled_bytes(M, K, ctypes.byref(b)))
    return b.value


def sp24_bench_dense_tile(W: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense bf16 W (M x K) -> its copy in v_mfma_f32_16x16x32_bf16 operand order (1-D bf16 buffer)."""
    _dev_check(W, out)
    M, K = W.shape
    nb = sp24_bench_dense_tiled_bytes(M, K)
    if out is None:
        out = torch.empty(nb // 2, dtype=torch.bfloat16, device=W.device)
    if out.numel() * 2 != nb or not out.is_contiguous():
        raise ValueError(f"the tiled copy needs a contiguous buffer of {nb} bytes")
    _check("sp24_bench_dense_tile", load_library().sp24_bench_dense_tile(_ptr(W), M, K, _rows(W, "W"), _ptr(out),
                                                                         _stream(W)))
    return out


def sp24_bench_gemm_dense_bf16(W_tiled: torch.Tensor, M: int, X: torch.Tensor, out_dtype: torch.dtype = torch.float32,
                               out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense token-major GEMM Y (N x M) = X (N x K) . W^T with the sparse tiled kernel's tiling (measurement only)."""
    _dev_check(W_tiled, X, out)
    N, K = X.shape
    if W_tiled.numel() * 2 != sp24_bench_dense_tiled_bytes(M, K):
        raise ValueError("W_tiled does not hold an M x K weight")
    if out is None:
        out = torch.empty((N, M), dtype=out_dtype, device=X.device)
    st = load_library().sp24_bench_gemm_dense_bf16(_ptr(W_tiled), M, K, _ptr(X), N, _rows(X, "X"), _ptr(out),
                                                   _TORCH_TO_SP24[out.dtype], _rows(out, "out"), _stream(X))
    _check("sp24_bench_gemm_dense_bf16", st)
    return out


def sp24_bench_stream_read(src: torch.Tensor, nbytes: int | None = None, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Streaming read of the first nbytes of src (measurement only); returns the per-workgroup XOR words
    (uint32, 4 per workgroup)."""
    _dev_check(src, sink)
    nb = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if nb > src.numel() * src.element_size() or not src.is_contiguous():
        raise ValueError("nbytes exceeds the contiguous source")
    lib = load_library()
    blocks = ctypes.c_int64()
    _check("sp24_bench_stream_read_blocks", lib.sp24_bench_stream_read_blocks(nb, ctypes.byref(blocks)))
    if sink is None:
        sink = torch.empty(4 * blocks.value, dtype=torch.int32, device=src.device)
    if sink.numel() * sink.element_size() < 16 * blocks.value:
        raise ValueError("sink too small")
    _check("sp24_bench_stream_read", lib.sp24_bench_stream_read(_ptr(src), nb, _ptr(sink), _stream(src)))
    return sink
