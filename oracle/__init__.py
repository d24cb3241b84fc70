"""sp24 CPU oracle -- TEST INFRASTRUCTURE ONLY.

numpy-facing wrapper around ``sp24_oracle.c``: a plain, slow, obviously correct CPU statement of the
2:4 structured-sparse path (column norms, prune + compress, decompress, sparse GEMM in bf16 and int8).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import it;
the product package never does, and this wrapper shares no code with the HIP path.

Pages (cited by title and section): the Orin NN design book, Chapter 7 "2:4 structured sparsity",
sections 2.1 (prune, values + 2-bit metadata, metadata mux), 5 (exercise Q1) and 6.1 (every 1x4 block
must hold 2 zeros); the zyxy.net Wanda lecture, section 2.1 (score = |w| * ||X_j||_2); the NVIDIA
technical blog on Ampere structured sparsity, Figure 1 (only non-zeros plus index metadata are stored).

Every function here is pinned by the ``-m "not gpu"`` tests against what the pages and arithmetic fix
(worked examples, brute force, closed forms, library routines); see tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sp24_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libsp24_oracle.so")

BF16, FP16, FP32, I8, I32 = 0, 1, 2, 3, 4
MAGNITUDE, WANDA = 0, 1
_DT_NP = {BF16: np.uint16, FP16: np.uint16, FP32: np.float32, I8: np.int8}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_col_norms.argtypes = [P, I64, I64, I64, P]
        lib.oracle_prune_compress.argtypes = [P, I, I64, I64, I64, I, P, P, I, P]
        lib.oracle_meta_check.argtypes = [P, I64, I64, I]
        lib.oracle_meta_check.restype = I64
        lib.oracle_compressed_bytes.argtypes = [I64, I64, I, ctypes.POINTER(I64), ctypes.POINTER(I64)]
        lib.oracle_values_offset.argtypes = [I64, I64, I64, I]
        lib.oracle_values_offset.restype = I64
        lib.oracle_meta_offset.argtypes = [I64, I64, I64, I]
        lib.oracle_meta_offset.restype = I64
        lib.oracle_decompress.argtypes = [P, P, I, I64, I64, P, I64]
        lib.oracle_prune_mask.argtypes = [P, I, I64, I64, I64, I, I, P, P, P, I64]
        lib.oracle_channel_permutation.argtypes = [P, I, I64, I64, I64, I, P, I, P]
        lib.oracle_retained.argtypes = [P, I, I64, I64, I64, I, P, P]
        lib.oracle_perm_pair.argtypes = [I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
        lib.oracle_perm_pair.restype = I
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = I
        lib.oracle_retained.restype = ctypes.c_double
        lib.oracle_gemm_bf16.argtypes = [P, P, I64, I64, P, I64, I64, P, I64, P]
        lib.oracle_gemm_i8.argtypes = [P, P, I64, I64, P, I64, I64, P, P, I64, P, P]
        lib.oracle_fp32_to_bf16.argtypes = [ctypes.c_float]
        lib.oracle_fp32_to_bf16.restype = ctypes.c_uint16
        lib.oracle_fp16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_fp16_value.restype = ctypes.c_double
        _lib = lib
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def col_norms(X_bf16: np.ndarray) -> np.ndarray:
    """norms[j] = ||X[j, :]||_2 (X: K x N bf16 bits as uint16, row pitch = stride)."""
    X = _c(X_bf16, np.uint16)
    K, N = X.shape
    ldx = X.strides[0] // 2 if K > 0 else N
    if X.strides[1] != 2:
        X = np.ascontiguousarray(X)
        ldx = N
    out = np.empty(K, np.float32)
    _check(_load().oracle_col_norms(_ptr(X), K, N, ldx, _ptr(out)))
    return out


_ESIZE = {BF16: 2, FP16: 2, FP32: 4, I8: 1}


def compressed_bytes(M: int, K: int, val_dtype: int):
    """(values bytes, metadata bytes) of the compressed form of an M x K weight."""
    vb, mb = ctypes.c_int64(), ctypes.c_int64()
    _check(_load().oracle_compressed_bytes(M, K, val_dtype, ctypes.byref(vb), ctypes.byref(mb)))
    return vb.value, mb.value


def prune_compress(W: np.ndarray, dtype: int, score: int = MAGNITUDE, norms: np.ndarray | None = None,
                   val_dtype: int | None = None):
    """Prune each group of 4 along K to its top-2 and compress. Returns (values, meta) as flat
    buffers in the tiled layout (values in val_dtype, meta uint8)."""
    val_dtype = dtype if val_dtype is None else val_dtype
    W = np.ascontiguousarray(_c(W, _DT_NP[dtype]))
    M, K = W.shape
    vb, mb = compressed_bytes(M, K, val_dtype)
    values = np.zeros(vb // _ESIZE[val_dtype], _DT_NP[val_dtype])
    meta = np.zeros(mb, np.uint8)
    if norms is not None:
        norms = np.ascontiguousarray(_c(norms, np.float32))
    _check(_load().oracle_prune_compress(_ptr(W), dtype, M, K, K, score, _ptr(norms), _ptr(values), val_dtype,
                                         _ptr(meta)))
    return values, meta


def prune_mask(W: np.ndarray, dtype: int, keep: int, score: int = MAGNITUDE, norms: np.ndarray | None = None):
    """k-of-4 mask (NVIDIA blog, progressive sparse training, Figure 4: keep 3 of 4, later 2 of 4).
    Returns (mask, masked): mask M x K/8 bytes (nibble of group g at byte g/2, even g low, bit t set
    when position t is kept) and the masked M x K weight (kept elements bit-copied, +0 elsewhere)."""
    W = np.ascontiguousarray(_c(W, _DT_NP[dtype]))
    M, K = W.shape
    mask = np.zeros((M, K // 8), np.uint8)
    out = np.zeros((M, K), _DT_NP[dtype])
    if norms is not None:
        norms = np.ascontiguousarray(_c(norms, np.float32))
    _check(_load().oracle_prune_mask(_ptr(W), dtype, M, K, K, keep, score, _ptr(norms), _ptr(mask), _ptr(out), K))
    return mask, out


def channel_permutation(W: np.ndarray, dtype: int, sweeps: int = 1, score: int = MAGNITUDE,
                        norms: np.ndarray | None = None) -> np.ndarray:
    """Input-channel permutation before pruning (Orin NN design, Chapter 7, section 3.1 Step 2 and
    section 6.3): the round-robin pair re-partition search of sp24_oracle.c. Returns perm (int32[K]):
    permuted column c is original column perm[c]."""
    W = np.ascontiguousarray(_c(W, _DT_NP[dtype]))
    M, K = W.shape
    perm = np.zeros(K, np.int32)
    if norms is not None:
        norms = np.ascontiguousarray(_c(norms, np.float32))
    _check(_load().oracle_channel_permutation(_ptr(W), dtype, M, K, K, score, _ptr(norms), sweeps, _ptr(perm)))
    return perm


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def perm_pair(G: int, r: int, p: int):
    """The pair of groups (ga < gb) that pair p of round r of a permutation sweep over G groups
    re-partitions, or None when one of the two positions is the dummy of an odd G."""
    a, b = ctypes.c_int(), ctypes.c_int()
    if not _load().oracle_perm_pair(int(G), int(r), int(p), ctypes.byref(a), ctypes.byref(b)):
        return None
    return a.value, b.value


def retained(W: np.ndarray, dtype: int, perm: np.ndarray | None = None, score: int = MAGNITUDE,
             norms: np.ndarray | None = None) -> float:
    """Sum over rows and groups of the two largest scores per group of the column order perm."""
    W = np.ascontiguousarray(_c(W, _DT_NP[dtype]))
    M, K = W.shape
    if perm is not None:
        perm = np.ascontiguousarray(np.asarray(perm, np.int32))
    if norms is not None:
        norms = np.ascontiguousarray(_c(norms, np.float32))
    return float(_load().oracle_retained(_ptr(W), dtype, M, K, K, score, _ptr(norms), _ptr(perm)))


def meta_bad_nibbles(meta: np.ndarray, M: int, K: int, val_dtype: int) -> int:
    meta = np.ascontiguousarray(_c(meta, np.uint8))
    return int(_load().oracle_meta_check(_ptr(meta), M, K, val_dtype))


def values_offset(i: int, b: int, K: int, val_dtype: int) -> int:
    return int(_load().oracle_values_offset(i, b, K, _ESIZE[val_dtype]))


def meta_offset(i: int, mb: int, K: int, val_dtype: int) -> int:
    return int(_load().oracle_meta_offset(i, mb, K, _ESIZE[val_dtype]))


def _check_sizes(values, meta, M, K, dtype):
    vb, mb = compressed_bytes(M, K, dtype)
    if values.nbytes != vb or meta.nbytes != mb:
        raise ValueError(f"compressed buffers of {values.nbytes}/{meta.nbytes} bytes, expected {vb}/{mb}")


def decompress(values: np.ndarray, meta: np.ndarray, dtype: int, M: int, K: int) -> np.ndarray:
    values = np.ascontiguousarray(_c(values, _DT_NP[dtype]))
    meta = np.ascontiguousarray(_c(meta, np.uint8))
    _check_sizes(values, meta, M, K, dtype)
    out = np.empty((M, K), _DT_NP[dtype])
    _check(_load().oracle_decompress(_ptr(values), _ptr(meta), dtype, M, K, _ptr(out), K))
    return out


def _rows_arg(rows, M):
    if rows is None:
        rows = np.arange(M, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def _feature_major(X: np.ndarray, layout: str) -> np.ndarray:
    """Token-major X (N x K, a Linear layer's input) holds the same numbers as feature-major X (K x N),
    transposed: the product is the same sum, only the storage order of its operands and result differs."""
    if layout == "feature":
        return X
    if layout == "token":
        return X.T
    raise ValueError(layout)


def gemm_bf16(values: np.ndarray, meta: np.ndarray, X: np.ndarray, M: int, rows=None,
              layout: str = "feature") -> np.ndarray:
    """Y[r, :] = (pruned W)[rows[r], :] . X in float64 (values/X: bf16 bits as uint16; K = X rows).
    layout "token": X is N x K and the result is returned N x len(rows) (Y[n, r])."""
    if layout != "feature":
        return gemm_bf16(values, meta, _feature_major(X, layout), M, rows).T
    values = np.ascontiguousarray(_c(values, np.uint16))
    meta = np.ascontiguousarray(_c(meta, np.uint8))
    X = np.ascontiguousarray(_c(X, np.uint16))
    K, N = X.shape
    _check_sizes(values, meta, M, K, BF16)
    r = _rows_arg(rows, M)
    Y = np.empty((len(r), N), np.float64)
    _check(_load().oracle_gemm_bf16(_ptr(values), _ptr(meta), M, K, _ptr(X), N, N, _ptr(r), len(r), _ptr(Y)))
    return Y


def gemm_i8(values: np.ndarray, meta: np.ndarray, X: np.ndarray, M: int, scale: np.ndarray | None = None,
            rows=None, layout: str = "feature"):
    """Exact int64 accumulators (checked to fit int32) and, with ``scale``, fl32(fl32(acc) * scale[m]).
    layout "token": X is N x K and both results are returned N x len(rows)."""
    if layout != "feature":
        acc, Y = gemm_i8(values, meta, _feature_major(X, layout), M, scale, rows)
        return acc.T, (None if Y is None else Y.T)
    values = np.ascontiguousarray(_c(values, np.int8))
    meta = np.ascontiguousarray(_c(meta, np.uint8))
    X = np.ascontiguousarray(_c(X, np.int8))
    K, N = X.shape
    _check_sizes(values, meta, M, K, I8)
    r = _rows_arg(rows, M)
    acc = np.empty((len(r), N), np.int64)
    Y = None
    if scale is not None:
        scale = np.ascontiguousarray(_c(scale, np.float32))
        Y = np.empty((len(r), N), np.float32)
    _check(_load().oracle_gemm_i8(_ptr(values), _ptr(meta), M, K, _ptr(X), N, N, _ptr(scale), _ptr(r), len(r),
                                  _ptr(acc), _ptr(Y)))
    return acc, Y


def gelu64(y) -> np.ndarray:
    """GELU(y) = y/2 (1 + erf(y / sqrt 2)) in float64 (the exact erf form used by BERT's FFN)."""
    from scipy.special import erf
    y = np.asarray(y, np.float64)
    return 0.5 * y * (1.0 + erf(y / np.sqrt(2.0)))


def requant_i8(y, out_scale: float) -> np.ndarray:
    """int8 code of y: clamp(rne(y * inv), -127, 127) with inv = fl32(1 / out_scale); fp32 inputs
    multiply in fp32 (one rounding), float64 inputs in float64."""
    y = np.asarray(y)
    inv = np.float32(1) / np.float32(out_scale)
    d = y * (inv if y.dtype == np.float32 else np.float64(inv))
    return np.clip(np.rint(d), -127, 127).astype(np.int8)


def gemm_i8_fused(values: np.ndarray, meta: np.ndarray, X: np.ndarray, M: int, scale: np.ndarray,
                  bias: np.ndarray | None = None, gelu: bool = False, out_scale: float | None = None, rows=None,
                  layout: str = "feature") -> dict:
    """The int8 GEMM's fused FFN epilogue (NVIDIA blog, quantization section: the sparse int8 BERT keeps
    its FFN in int8; oeforum post: int8 and 2:4 combine), step by step in the pages' order:
      y32 = fl32(fl32(acc) * scale[m])      (gemm_i8)
      y32 = fl32(y32 + bias[m])             (fp32 add, when bias is given)
      y   = GELU(y32)                       (float64 reference, when gelu)
      q   = clamp(rne(y * fl32(1/out_scale)))  (fp32 multiply without GELU; float64 with it)
    Returns dict(y32=..., y=..., q=...) laid out as gemm_i8's results for the layout."""
    _, y32 = gemm_i8(values, meta, X, M, scale, rows=rows, layout=layout)
    if bias is not None:
        b = np.asarray(bias, np.float32)[_rows_arg(rows, M)]
        y32 = (y32 + (b[None, :] if layout == "token" else b[:, None])).astype(np.float32)
    y = gelu64(y32) if gelu else y32
    q = requant_i8(y, out_scale) if out_scale is not None else None
    return dict(y32=y32, y=y, q=q)


def fp32_to_bf16(x: float) -> int:
    return int(_load().oracle_fp32_to_bf16(float(x)))


def fp16_value(h: int) -> float:
    return float(_load().oracle_fp16_value(int(h)))
