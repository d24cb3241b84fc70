"""Helpers for the GPU parity tests: moving numpy bit patterns to and from device tensors, and the
comparison rules (bit-exact for selection/metadata/integers; Frobenius and element bounds for bf16)."""
import os
import sys

import numpy as np
import pytest
import torch

_TO_TORCH = {np.uint16: torch.bfloat16, np.float32: torch.float32, np.int8: torch.int8, np.uint8: torch.uint8,
             np.int32: torch.int32}


def say(msg: str):
    """Name the case before a GPU step (flushed, so it survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    import structured_sparse_gemm_sp24_amd as sp
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    if not os.path.exists(sp.LIB_PATH):
        pytest.fail("libsp24.so is not built; build before running GPU tests")
    sp.load_library()


def dev(a: np.ndarray, kind: str | None = None) -> torch.Tensor:
    """numpy -> device tensor. kind 'bf16'/'fp16' reinterprets uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if kind == "fp16":
        return torch.from_numpy(a.view(np.int16)).view(torch.float16).cuda()
    return torch.from_numpy(a).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy, 16-bit floats as uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def frob_rel(y: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm((y.astype(np.float64) - ref).ravel())
    n = np.linalg.norm(ref.ravel())
    return float(d / n) if n > 0 else float(d)


def fp32_sum_bound(absprod_sum: np.ndarray, K: int) -> np.ndarray:
    """Worst-case error of summing K exact products in fp32 in any order: K * 2^-24 * sum |w x|
    (plus a tiny absolute term for underflow)."""
    return K * 2.0 ** -24 * absprod_sum + 1e-30


def rne_bf16_from_f64(y: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 bit patterns (through float32, then nearest even). The two
    roundings can differ from one direct rounding by one bf16 ulp in rare halfway cases, so this is
    only used under the Frobenius gate."""
    f = torch.from_numpy(np.ascontiguousarray(y.astype(np.float32)))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
