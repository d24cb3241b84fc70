"""Benchmark of the 2:4 sparse hot path on one MI355X.

One step = one pass of a workload's whole path over its synthetic batch. The default workload is the
largest single-GPU configuration: the 28672 x 8192 FFN projection at N = 8192 tokens -- 2:4 magnitude
prune + compress of W (bf16), then the sparse GEMM of the 8192 tokens (bf16 in and out), token-major as
a Linear layer holds its activations (X 8192 x 8192, Y 8192 x 28672); --layout feature uses X K x N and
Y M x N instead (the same products). Other workloads (--workload, --n) cover the single 256 x 256 Linear,
the ViT-B/16 MLP fc1 layer, the BERT-base int8 FFN pair (also as one fused int8 chain), the LLM
projections with Wanda scoring, int8 decoding of a few tokens, and the FFN at N = 8 / 64 / 512. Inputs
are resident in HBM before timing; steps rotate over enough copies of every buffer that each kernel's
launches cycle over more than twice the 256 MB Infinity Cache (within a memory budget), so each launch
reads its operands from HBM. The roofline also carries the sustained shader clock under matrix-core
load (sp24_probe_sclk) and the MFMA peak scaled to it.

Prints ONE JSON line: the step's dense-equivalent throughput (2*M*N*K per GEMM), the dominant
kernel's roofline (its average duration from HIP events on the launch stream; algorithmic bytes or
flops per launch; HBM traffic from the committed counter summary when the kernel source matches),
per-kernel averages, per-launch median / p10 / p90 and warm (one copy, cache-resident) averages, and
the CPU oracle timed per function on the GPU machine's host on a bounded sample of the same workload. The
timed steps, and the repeated launches behind each kernel's average, are replayed from HIP graphs, so
microsecond kernels are timed without the Python binding's per-call overhead between them.

Roofline conventions: a 2:4 GEMM executes M*N*K/2 multiply-adds, i.e. M*N*K algorithmic flops, which
are priced against the dense MFMA peak of the dtype (bf16 2516.6 TFLOP/s, int8 5033.2 TOP/s); this
fraction equals the dense-equivalent rate 2*M*N*K/t over the sparse-MFMA peak. HBM-bound kernels are
priced as algorithmic bytes / t against 8 TB/s. A kernel whose epilogue's VALU work outweighs both (the fused
int8 GEMM with GELU) is priced as its VALU lane-instruction slots / t against the issue rate
256 x 4 x 16 x 2.4 GHz = 39.3 Tslot/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import structured_sparse_gemm_sp24_amd as sp  # noqa: E402
from structured_sparse_gemm_sp24_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
DENSE_PEAK = {"bf16": 2516.6, "i8": 5033.2}   # TFLOP/s (bf16) and TOP/s (int8), dense MFMA
# VALU issue rate in lane-instruction slots per second: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz
# (unpacked fp32; a transcendental takes 4 slots)
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# slots per output of the fused int8 epilogue with GELU and int8 output: dequant (convert, scale, bias: 3),
# GELU by Abramowitz & Stegun 7.1.26 (13 full-rate + reciprocal and exp2 at 4 slots each: 21), requantization
# (scale, round by adding 1.5 * 2^23, clamp: 3), one slot for packing four codes
GELU_I8_SLOTS_PER_OUTPUT = 28
SPEC_SCLK_MHZ = 2400.0                          # the clock those peaks are quoted at
CACHE_BYTES = 256 << 20                      # MI355X Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "structured_sparse_gemm_sp24_amd", "csrc")
TILED_MIN_N = 65                             # sp24_gemm_bf16 uses the LDS-tiled kernel above N = 64


def to_dev(a, kind=None):
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def n_copies(step_bytes: int, kernel_bytes: int, budget: int = 8 << 30) -> int:
    """Buffer copies to rotate so that every kernel's launches cycle over more than twice the Infinity
    Cache (kernel_bytes: the smallest bytes one kernel of the step touches), within a memory budget, and
    never fewer than three (each launch then follows launches on two other copies)."""
    n = int(np.ceil(2 * CACHE_BYTES / max(kernel_bytes, 1))) + 1
    return max(3, min(64, n, budget // max(step_bytes, 1)))


class Kernel:
    """One launch of the step: fn(copy), algorithmic bytes and flops per launch, the dtype of its
    arithmetic, and the source files whose digest keys its counter-measured traffic."""

    def __init__(self, name, fn, nbytes, flops=0.0, dtype="bf16", sources=(), valu_slots=0.0):
        self.name, self.fn, self.nbytes, self.flops, self.dtype, self.sources = name, fn, nbytes, flops, dtype, sources
        self.valu_slots = valu_slots  # VALU lane-instruction slots the epilogue's definition takes (0: none)


def gemm_sources(N):
    """Sources of the bf16 GEMM kernels that can run at N tokens (the library picks among them by shape)."""
    if N >= TILED_MIN_N:
        return ("gemm_bf16_tiled.hip", "sp24_device.h")
    return ("gemm_bf16_fewtok.hip", "gemm_bf16_skinny.hip", "sp24_device.h")


# ----------------------------------------------------------------------------- oracle timing helpers

def _median_s(fn, reps=3):
    """Median wall time of `reps` calls of fn()."""
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def _gemm_rows_timed(run, M, budget_s, first_rows):
    """Time the oracle GEMM on a leading row slice sized to about budget_s. The oracle spreads rows over its
    threads, so two short runs of 2T and 6T rows (T threads; at least first_rows) give the fixed part
    (operand conversion, metadata check) and the per-row cost; a third run takes as many whole rounds of T
    rows as fit the budget. Returns (seconds scaled to all M rows, rows timed, extrapolated?)."""
    import oracle
    T = max(oracle.threads(), 1)
    r0 = min(M, max(first_rows, 2 * T))
    t0 = time.perf_counter()
    run(r0)
    t_small = time.perf_counter() - t0
    if r0 == M:
        return t_small, M, False
    r1 = min(M, 3 * r0)
    t0 = time.perf_counter()
    run(r1)
    t_big = time.perf_counter() - t0
    if r1 == M:
        return t_big, M, False
    per_row = max((t_big - t_small) / (r1 - r0), 1e-7)
    fixed = max(t_small - per_row * r0, 0.0)
    rows = int(min(M, max(r1, (budget_s - fixed) / per_row) // T * T))
    if fixed + per_row * M <= budget_s:
        rows = M
    if rows > r1:
        t0 = time.perf_counter()
        run(rows)
        t_rows = time.perf_counter() - t0
    else:
        rows, t_rows = r1, t_big
    if rows >= M:
        return t_rows, M, False
    fixed = min(fixed, t_rows)
    return fixed + (t_rows - fixed) * M / rows, rows, True


def _fn_entry(seconds, nbytes=None, flops=None, extrapolated=False, rows=None, total_rows=None):
    e = dict(s=round(seconds, 4))
    if nbytes:
        e["gbs"] = round(nbytes / seconds / 1e9, 3)
    if flops:
        e["gflops_dense_equiv"] = round(2 * flops / seconds / 1e9, 3)
    if extrapolated:
        e["extrapolated"] = f"timed on the first {rows} of {total_rows} rows, scaled to all rows"
    return e


# ----------------------------------------------------------------------------- workloads
# Each builder returns: name, config, dtype, flops (dense-equivalent per step), copies, kernels (in
# step order), dense_ref (optional: the dense GEMM of the same shape), cpu_sample(budget) -> (step seconds,
# what was timed, per-function timings).

def _bf16_gemm_workload(name, W_host, X_host, score, Xcal_host, config, layout, out=torch.bfloat16):
    """X_host is K x N (feature-major); with layout 'token' the device copies hold X^T (N x K) and Y is
    N x M."""
    M, K = W_host.shape
    N = X_host.shape[1]
    tm = layout == "token"
    config = dict(config, layout="token-major: X N x K, Y N x M" if tm else "feature-major: X K x N, Y M x N")
    X_dev_host = np.ascontiguousarray(X_host.T) if tm else X_host
    vb, mb = sp.sp24_compressed_bytes(M, K, torch.bfloat16)
    ob = 2 if out == torch.bfloat16 else 4
    step_bytes = M * K * 2 + vb + mb + K * N * 2 + M * N * ob + (Xcal_host.size * 2 if Xcal_host is not None else 0)
    kernel_bytes = min(M * K * 2 + vb + mb, vb + mb + K * N * 2 + M * N * ob,
                       Xcal_host.size * 2 if Xcal_host is not None else step_bytes)
    copies = []
    for _ in range(n_copies(step_bytes, kernel_bytes)):
        c = dict(W=to_dev(W_host, "bf16"), X=to_dev(X_dev_host, "bf16"),
                 vals=torch.empty(vb // 2, dtype=torch.bfloat16, device="cuda"),
                 meta=torch.empty(mb, dtype=torch.uint8, device="cuda"),
                 Y=torch.empty((N, M) if tm else (M, N), dtype=out, device="cuda"))
        if Xcal_host is not None:
            c["Xcal"] = to_dev(Xcal_host, "bf16")
            c["norms"] = torch.empty(K, dtype=torch.float32, device="cuda")
        copies.append(c)
    kernels = []
    if Xcal_host is not None:
        Ncal = Xcal_host.shape[1]
        kernels.append(Kernel("col_norms", lambda c: sp.sp24_col_norms(c["Xcal"], norms=c["norms"]),
                              K * Ncal * 2 + K * 4, sources=("norms.hip", "sp24_device.h")))
    wanda = score == sp.SP24_SCORE_WANDA
    kernels.append(Kernel(
        "prune_compress",
        lambda c: sp.sp24_prune_compress(c["W"], score=score, norms=c["norms"] if wanda else None, values=c["vals"],
                                         meta=c["meta"]),
        M * K * 2 + (K * 4 if wanda else 0) + M * K * 9 // 8, sources=("prune.hip", "sp24_device.h")))
    lay = "token" if tm else "feature"
    kernels.append(Kernel("gemm_bf16",
                          lambda c: sp.sp24_gemm_bf16_ex(c["vals"], c["meta"], M, c["X"], layout=lay, out=c["Y"]),
                          M * K * 9 // 8 + K * N * 2 + M * N * ob, float(M) * N * K, "bf16", gemm_sources(N)))

    def dense_ref():
        """Dense bf16 GEMMs of the same shape on the decompressed (pruned) weight: hipBLASLt through
        torch.matmul, and (token-major, K % 64 == 0) the library's dense reference with the sparse tiled
        kernel's tiling (include/sp24_bench.h)."""
        c0 = copies[0]
        for k in kernels:
            k.fn(c0)
        Wd = sp.sp24_decompress(c0["vals"], c0["meta"], M, K)
        out = {}
        if tm:
            Wtr = Wd.t()  # X (N x K) @ W^T, the Linear layer's own product
            Yd = torch.empty((N, M), dtype=torch.bfloat16, device="cuda")
            out["dense_bf16_matmul_same_shape"] = lambda c: torch.matmul(c["X"], Wtr, out=Yd)
            if K % 64 == 0 and N >= TILED_MIN_N:
                Wtiled = sp.sp24_bench_dense_tile(Wd)
                out["dense_bf16_same_tiling"] = lambda c: sp.sp24_bench_gemm_dense_bf16(Wtiled, M, c["X"], out=Yd)
        else:
            Yd = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            out["dense_bf16_matmul_same_shape"] = lambda c: torch.matmul(Wd, c["X"], out=Yd)
        return out

    def cpu_sample(budget_s):
        """The oracle per function: column norms, prune/compress and decompress of the whole weight (median
        of 3), and the GEMM on a leading row slice sized to the budget, scaled to all rows. The step is
        norms + prune/compress + GEMM."""
        import oracle
        per = {}
        sc = oracle.WANDA if wanda else oracle.MAGNITUDE
        norms = None
        if Xcal_host is not None:
            norms = oracle.col_norms(Xcal_host)
            per["col_norms"] = _fn_entry(_median_s(lambda: oracle.col_norms(Xcal_host)), nbytes=Xcal_host.size * 2 + K * 4)
        v, m = oracle.prune_compress(W_host, oracle.BF16, sc, norms)
        per["prune_compress"] = _fn_entry(_median_s(lambda: oracle.prune_compress(W_host, oracle.BF16, sc, norms)),
                                          nbytes=M * K * 2 + M * K * 9 // 8)
        per["decompress"] = _fn_entry(_median_s(lambda: oracle.decompress(v, m, oracle.BF16, M, K)),
                                      nbytes=M * K * 9 // 8 + M * K * 2)
        t_gemm, rows, extra = _gemm_rows_timed(
            lambda r: oracle.gemm_bf16(v, m, X_dev_host, M, rows=np.arange(r), layout=lay), M,
            max(budget_s - sum(e["s"] for e in per.values()), 1.0), 8)
        per["gemm_bf16"] = _fn_entry(t_gemm, flops=float(M) * N * K, extrapolated=extra, rows=rows, total_rows=M)
        total = t_gemm + per["prune_compress"]["s"] + (per["col_norms"]["s"] if "col_norms" in per else 0.0)
        what = ("column norms + " if norms is not None else "") + f"prune/compress of the full {M}x{K} W (median of 3)"
        gemm_what = f"GEMM on the first {rows} of {M} rows (N = {N}), scaled to all rows" if extra else f"GEMM on all {M} rows"
        return total, f"{what} + {gemm_what}", per

    return dict(name=name if tm else name + "_feature", dtype="bf16", unit="TFLOP/s", config=config,
                flops=2.0 * M * N * K, copies=copies, kernels=kernels, dense_ref=dense_ref, cpu_sample=cpu_sample)


def workload_vit(args):
    d = synth.vit_b16_fc1()
    M, K = d["W_bf16"].shape
    N = d["X_bf16"].shape[1]
    cfg = dict(workload="vit_b16_fc1", M=M, K=K, N=N, weight="bf16 N(0,0.02^2) seed 11",
               activations="bf16 N(0,1) seed 12, N = 32 images x 197 tokens", score="magnitude", out="bf16",
               step="prune_compress + gemm_bf16")
    return _bf16_gemm_workload("vit_b16_fc1", d["W_bf16"], d["X_bf16"], sp.SP24_SCORE_MAGNITUDE, None, cfg, args.layout)


def shard_rows(W, args, cfg, name):
    """--shard-m G: one GPU's share of the layer split by output channels over G GPUs (rows [0, M/G) rounded up
    to whole 16-row blocks); every GPU of such a split streams its own rows with no exchange."""
    G = args.shard_m
    if G == 1:
        return W, cfg, name
    M = W.shape[0]
    Mg = -(-M // G // 16) * 16 if M % (16 * G) else M // G
    cfg = dict(cfg, M=Mg, shard=f"rows [0, {Mg}) of {M}: one GPU's share of an output-channel split over {G} GPUs")
    return np.ascontiguousarray(W[:Mg]), cfg, f"{name}_mshard{G}"


def workload_llm(M):
    def build(args):
        N = args.n or 4096
        d = synth.llm_proj(M)
        X = np.ascontiguousarray(d["X_bf16"][:, :N])
        cfg = dict(workload=f"llm_proj_{M}x4096", M=M, K=4096, N=N,
                   weight=f"bf16 N(0,0.02^2) seed {31 if M == 11008 else 32}",
                   calibration="4096 x 2048 bf16, lognormal(0,1) channel scale x Student-t(3), seed 33",
                   activations="same law, seed 34, first N columns", score="wanda", out="bf16",
                   step="col_norms + prune_compress (Wanda) + gemm_bf16")
        W, cfg, name = shard_rows(d["W_bf16"], args, cfg, f"llm_proj_{M}x4096_n{N}")
        return _bf16_gemm_workload(name, W, X, sp.SP24_SCORE_WANDA, d["Xcal_bf16"], cfg, args.layout)
    return build


def workload_ffn(args):
    N = args.n or 8192
    d = synth.ffn_28672x8192(N)
    cfg = dict(workload="ffn_28672x8192", M=28672, K=8192, N=N, weight="bf16 N(0,0.02^2) seed 41",
               activations="bf16 N(0,1) seed 42, first N columns of an 8192-wide draw", score="magnitude",
               out="bf16", step="prune_compress + gemm_bf16")
    W, cfg, name = shard_rows(d["W_bf16"], args, cfg, f"ffn_28672x8192_n{N}")
    return _bf16_gemm_workload(name, W, d["X_bf16"], sp.SP24_SCORE_MAGNITUDE, None, cfg, args.layout)


def workload_single(args):
    d = synth.single_linear_256()
    W, X = d["W_f32"], d["X_bf16"]
    M, K = W.shape
    N = X.shape[1]
    vb, mb = sp.sp24_compressed_bytes(M, K, torch.bfloat16)
    tm = args.layout == "token"
    Xdev = np.ascontiguousarray(X.T) if tm else X
    copies = [dict(W=to_dev(W), X=to_dev(Xdev, "bf16"), vals=torch.empty(vb // 2, dtype=torch.bfloat16, device="cuda"),
                   meta=torch.empty(mb, dtype=torch.uint8, device="cuda"),
                   Y=torch.empty((N, M) if tm else (M, N), dtype=torch.float32, device="cuda")) for _ in range(8)]
    kernels = [
        Kernel("prune_compress", lambda c: sp.sp24_prune_compress(c["W"], val_dtype=torch.bfloat16, values=c["vals"],
                                                                  meta=c["meta"]),
               M * K * 4 + M * K * 9 // 8, sources=("prune.hip", "sp24_device.h")),
        Kernel("gemm_bf16", lambda c: sp.sp24_gemm_bf16_ex(c["vals"], c["meta"], M, c["X"], layout=args.layout,
                                                           out=c["Y"]),
               M * K * 9 // 8 + K * N * 2 + M * N * 4, float(M) * N * K, "bf16", gemm_sources(N))]

    def cpu_sample(budget_s):
        import oracle
        v, m = oracle.prune_compress(W, oracle.FP32, val_dtype=oracle.BF16)
        per = dict(prune_compress=_fn_entry(_median_s(lambda: oracle.prune_compress(W, oracle.FP32, val_dtype=oracle.BF16)),
                                            nbytes=M * K * 4 + M * K * 9 // 8),
                   decompress=_fn_entry(_median_s(lambda: oracle.decompress(v, m, oracle.BF16, M, K)),
                                        nbytes=M * K * 9 // 8 + M * K * 2),
                   gemm_bf16=_fn_entry(_median_s(lambda: oracle.gemm_bf16(v, m, X, M)), flops=float(M) * N * K))
        return (per["prune_compress"]["s"] + per["gemm_bf16"]["s"],
                "the whole step (prune/compress fp32 -> bf16 values, GEMM), median of 3", per)

    cfg = dict(workload="single_linear_256", M=M, K=K, N=N, weight="fp32 N(0,1) seed 1, kept values rounded to bf16",
               activations="fp32 N(0,1) seed 2 rounded to bf16", score="magnitude", out="fp32",
               step="prune_compress + gemm_bf16",
               layout="token-major: X N x K, Y N x M" if tm else "feature-major: X K x N, Y M x N")
    return dict(name="single_linear_256", dtype="bf16", unit="TFLOP/s", config=cfg, flops=2.0 * M * N * K,
                copies=copies, kernels=kernels, dense_ref=None, cpu_sample=cpu_sample)


def workload_bert_int8(args):
    """BERT-base FFN pair in int8: W1 3072x768 and W2 768x3072 magnitude-pruned 2:4 in fp32, then per-row
    symmetric int8 (99.99 % coverage); activations per-tensor int8. The step prunes/compresses both
    int8 weights on the GPU and runs both int8 GEMMs (int32 accumulate, fp32 dequant epilogue)."""
    d = synth.bert_ffn_int8_dense()
    layers = []
    for wk, xk in (("W1_f32", "X1_f32"), ("W2_f32", "X2_f32")):
        Wf = d[wk]
        M, K = Wf.shape
        # host data prep (untimed): prune the fp32 weight with the library itself, then quantize
        v, m = sp.sp24_prune_compress(to_dev(Wf))
        Wp = sp.sp24_decompress(v, m, M, K).cpu().numpy()
        q, s_w = synth.quantize_rows(Wp)
        xq, s_x = synth.quantize_tensor(d[xk])
        xdev = np.ascontiguousarray(xq.T) if args.layout == "token" else xq
        layers.append(dict(M=M, K=K, N=xq.shape[1], q=q, xq=xq, xdev=xdev, scale=synth.dequant_scales(s_w, s_x)))
    step_bytes = sum(L["M"] * L["K"] * 2 + L["K"] * L["N"] + 4 * L["M"] * L["N"] for L in layers)
    # the smallest kernel: an int8 prune/compress (M K read, 5/8 M K written)
    kernel_bytes = min(L["M"] * L["K"] * 13 // 8 for L in layers)
    copies = []
    for _ in range(n_copies(step_bytes, kernel_bytes)):
        c = {}
        for i, L in enumerate(layers):
            vb, mb = sp.sp24_compressed_bytes(L["M"], L["K"], torch.int8)
            ysh = (L["N"], L["M"]) if args.layout == "token" else (L["M"], L["N"])
            c[i] = dict(W=to_dev(L["q"]), X=to_dev(L["xdev"]), scale=to_dev(L["scale"]),
                        vals=torch.empty(vb, dtype=torch.int8, device="cuda"),
                        meta=torch.empty(mb, dtype=torch.uint8, device="cuda"),
                        Y=torch.empty(ysh, dtype=torch.float32, device="cuda"))
        copies.append(c)
    kernels = []
    for i, L in enumerate(layers):
        M, K, N = L["M"], L["K"], L["N"]
        kernels.append(Kernel(f"prune_compress_i8_w{i + 1}",
                              lambda c, i=i: sp.sp24_prune_compress(c[i]["W"], values=c[i]["vals"], meta=c[i]["meta"]),
                              M * K + M * K * 5 // 8, sources=("prune.hip", "sp24_device.h")))
        kernels.append(Kernel(f"gemm_i8_w{i + 1}",
                              lambda c, i=i, M=M: sp.sp24_gemm_i8_ex(c[i]["vals"], c[i]["meta"], M, c[i]["X"],
                                                                     scale=c[i]["scale"], layout=args.layout,
                                                                     out=c[i]["Y"]),
                              M * K * 5 // 8 + K * N + 4 * M * N + 4 * M, float(M) * N * K, "i8",
                              ("gemm_i8_tiled_impl.h", "gemm_i8_tiled.hip", "sp24_device.h")))

    def cpu_sample(budget_s):
        import oracle
        total, parts, per = 0.0, [], {}
        for i, L in enumerate(layers):
            M, K = L["M"], L["K"]
            v8, m8 = oracle.prune_compress(L["q"], oracle.I8)
            e = _fn_entry(_median_s(lambda L=L: oracle.prune_compress(L["q"], oracle.I8)), nbytes=M * K * 13 // 8)
            per[f"prune_compress_i8_w{i + 1}"] = e
            per[f"decompress_i8_w{i + 1}"] = _fn_entry(_median_s(lambda v8=v8, m8=m8, M=M, K=K: oracle.decompress(v8, m8, oracle.I8, M, K)),
                                                       nbytes=M * K * 13 // 8)
            t, rows, extra = _gemm_rows_timed(
                lambda r, L=L, v8=v8, m8=m8: oracle.gemm_i8(v8, m8, L["xq"], L["M"], L["scale"], rows=np.arange(r)),
                M, max(budget_s / 2 - e["s"], 0.5), 16)
            per[f"gemm_i8_w{i + 1}"] = _fn_entry(t, flops=float(M) * L["N"] * K, extrapolated=extra, rows=rows, total_rows=M)
            total += e["s"] + t
            parts.append(f"{M}x{K}: GEMM on {rows} rows" + (", scaled to all rows" if extra else ""))
        return total, "int8 prune/compress of both weights (median of 3) + " + ", ".join(parts), per

    cfg = dict(workload="bert_ffn_int8", W1="3072x768", W2="768x3072", N=8192,
               weights="fp32 N(0,0.02^2) seeds 21/22, 2:4 magnitude, per-row int8 at 99.99 % coverage",
               activations="fp32 N(0,1) seeds 23/24, per-tensor int8 at 99.99 % coverage (64 x 128 tokens)",
               out="fp32 (int32 accumulate, per-channel dequant)", step="2 x (prune_compress int8 + gemm_i8)",
               layout="token-major: X N x K, Y N x M" if args.layout == "token" else "feature-major: X K x N, Y M x N")
    flops = sum(2.0 * L["M"] * L["N"] * L["K"] for L in layers)
    return dict(name="bert_ffn_int8" + ("" if args.layout == "token" else "_feature"), dtype="i8", unit="TOP/s",
                config=cfg, flops=flops, copies=copies,
                kernels=kernels, dense_ref=None, cpu_sample=cpu_sample)


def workload_bert_int8_fused(args):
    """The BERT-base FFN as one int8 chain: H = int8(GELU(W1 X + b1)) from the fused epilogue of the
    first GEMM (requantized at the hidden activations' scale), then Y = W2 H + b2 in fp32. Weights and
    input are prepared as in bert_ffn_int8; the hidden scale is the 99.99 % coverage scale of
    GELU(W1 X + b1), found once before timing. The step prunes/compresses both int8 weights and runs
    both fused GEMMs."""
    d = synth.bert_ffn_int8_dense()
    bias = synth.bert_ffn_biases()
    tm = args.layout == "token"
    lay = "token" if tm else "feature"
    qw = []
    for wk in ("W1_f32", "W2_f32"):
        Wf = d[wk]
        M, K = Wf.shape
        v, m = sp.sp24_prune_compress(to_dev(Wf))
        q, s_w = synth.quantize_rows(sp.sp24_decompress(v, m, M, K).cpu().numpy())
        qw.append((q, s_w))
    xq, s_x = synth.quantize_tensor(d["X1_f32"])
    N = xq.shape[1]
    xdev = np.ascontiguousarray(xq.T) if tm else xq
    (q1, s_w1), (q2, s_w2) = qw
    M1, K1 = q1.shape
    M2, K2 = q2.shape
    scale1 = synth.dequant_scales(s_w1, s_x)
    # hidden activation scale (host prep, untimed): one fp32 pass of the first fused GEMM
    v1, m1 = sp.sp24_prune_compress(to_dev(q1))
    Hf = sp.sp24_gemm_i8_fused(v1, m1, M1, to_dev(xdev), to_dev(scale1), bias=to_dev(bias["b1"]), activation="gelu",
                               layout=lay).cpu().numpy()
    s_h = float(np.float32(np.quantile(np.abs(Hf.astype(np.float64)), 0.9999) / 127.0))
    scale2 = synth.dequant_scales(s_w2, np.float32(s_h))
    del Hf
    hsh = (N, M1) if tm else (M1, N)
    ysh = (N, M2) if tm else (M2, N)
    step_bytes = M1 * K1 * 2 + M2 * K2 * 2 + K1 * N + 2 * M1 * N + 4 * M2 * N
    kernel_bytes = min(M1 * K1 * 13 // 8, M2 * K2 * 13 // 8)
    copies = []
    for _ in range(n_copies(step_bytes, kernel_bytes)):
        c = dict(W1=to_dev(q1), W2=to_dev(q2), X=to_dev(xdev), s1=to_dev(scale1), s2=to_dev(scale2),
                 b1=to_dev(bias["b1"]), b2=to_dev(bias["b2"]),
                 H=torch.empty(hsh, dtype=torch.int8, device="cuda"),
                 Y=torch.empty(ysh, dtype=torch.float32, device="cuda"))
        for i, (M, K) in enumerate(((M1, K1), (M2, K2))):
            vb, mb = sp.sp24_compressed_bytes(M, K, torch.int8)
            c[f"v{i}"] = torch.empty(vb, dtype=torch.int8, device="cuda")
            c[f"m{i}"] = torch.empty(mb, dtype=torch.uint8, device="cuda")
        copies.append(c)
    srcs = ("gemm_i8_tiled_impl.h", "gemm_i8_tiled_i8.hip", "sp24_device.h")
    kernels = [
        Kernel("prune_compress_i8_w1", lambda c: sp.sp24_prune_compress(c["W1"], values=c["v0"], meta=c["m0"]),
               M1 * K1 + M1 * K1 * 5 // 8, sources=("prune.hip", "sp24_device.h")),
        Kernel("prune_compress_i8_w2", lambda c: sp.sp24_prune_compress(c["W2"], values=c["v1"], meta=c["m1"]),
               M2 * K2 + M2 * K2 * 5 // 8, sources=("prune.hip", "sp24_device.h")),
        Kernel("gemm_i8_w1_gelu_i8out",
               lambda c: sp.sp24_gemm_i8_fused(c["v0"], c["m0"], M1, c["X"], c["s1"], bias=c["b1"], activation="gelu",
                                               out_dtype=torch.int8, out_scale=s_h, layout=lay, out=c["H"]),
               M1 * K1 * 5 // 8 + K1 * N + M1 * N + 8 * M1, float(M1) * N * K1, "i8", srcs,
               valu_slots=float(GELU_I8_SLOTS_PER_OUTPUT) * M1 * N),
        Kernel("gemm_i8_w2_bias_f32out",
               lambda c: sp.sp24_gemm_i8_fused(c["v1"], c["m1"], M2, c["H"], c["s2"], bias=c["b2"], layout=lay,
                                               out=c["Y"]),
               M2 * K2 * 5 // 8 + K2 * N + 4 * M2 * N + 8 * M2, float(M2) * N * K2, "i8",
               ("gemm_i8_tiled_impl.h", "gemm_i8_tiled.hip", "sp24_device.h")),
    ]

    def cpu_sample(budget_s):
        import oracle
        per = {}
        v8, m8 = oracle.prune_compress(q1, oracle.I8)
        per["prune_compress_i8_w1"] = _fn_entry(_median_s(lambda: oracle.prune_compress(q1, oracle.I8)), nbytes=M1 * K1 * 13 // 8)
        per["prune_compress_i8_w2"] = _fn_entry(_median_s(lambda: oracle.prune_compress(q2, oracle.I8)), nbytes=M2 * K2 * 13 // 8)
        t1, rows, extra = _gemm_rows_timed(
            lambda r: oracle.gemm_i8_fused(v8, m8, xq, M1, scale1, bias["b1"], gelu=True, out_scale=s_h, rows=np.arange(r)),
            M1, max(budget_s - per["prune_compress_i8_w1"]["s"] - per["prune_compress_i8_w2"]["s"], 0.5), 16)
        per["gemm_i8_w1_gelu_i8out"] = _fn_entry(t1, flops=float(M1) * N * K1, extrapolated=extra, rows=rows, total_rows=M1)
        # the second GEMM has the same multiply-add count as the first
        total = per["prune_compress_i8_w1"]["s"] + per["prune_compress_i8_w2"]["s"] + 2 * t1
        return total, (f"int8 prune/compress of both weights (median of 3) + fused GEMM 1 on {rows} of {M1} rows, "
                       "scaled to all rows and doubled for GEMM 2 (same multiply-adds)"), per

    cfg = dict(workload="bert_ffn_int8_fused", W1="3072x768", W2="768x3072", N=N,
               weights="fp32 N(0,0.02^2) seeds 21/22, 2:4 magnitude, per-row int8 at 99.99 % coverage",
               biases="fp32 N(0,0.02^2) seeds 25/26",
               activations="fp32 N(0,1) seed 23, per-tensor int8 at 99.99 % coverage (64 x 128 tokens)",
               hidden=f"int8 codes of GELU(W1 X + b1) at scale {s_h:.6g} (99.99 % coverage)",
               out="fp32 W2 H + b2", step="2 x prune_compress int8 + fused GEMM 1 (bias, GELU, int8 out) + "
                                       "fused GEMM 2 (bias, fp32 out)",
               layout="token-major: X N x K, Y N x M" if tm else "feature-major: X K x N, Y M x N")
    flops = 2.0 * M1 * N * K1 + 2.0 * M2 * N * K2
    return dict(name="bert_ffn_int8_fused" + ("" if tm else "_feature"), dtype="i8", unit="TOP/s", config=cfg,
                flops=flops, copies=copies,
                kernels=kernels, dense_ref=None, cpu_sample=cpu_sample)


def workload_llm_int8(args):
    """An LLM projection decoding a few tokens in int8: W 11008x4096 magnitude-pruned 2:4 in fp32, then
    per-row symmetric int8 (99.99 % coverage); N tokens (default 16, at most 64) per-tensor int8. The step
    prunes/compresses the int8 weight on the GPU and runs the int8 GEMM (int32 accumulate, fp32 dequant),
    token-major, which for N <= 64 streams the 28 MB compressed weight once."""
    N = args.n or 16
    if not 1 <= N <= 64:
        raise SystemExit("llm_proj_11008x4096_int8: --n must be in 1..64")
    d = synth.llm_proj_int8_dense()
    Wf = d["W_f32"]
    M, K = Wf.shape
    # host data prep (untimed): prune the fp32 weight with the library itself, then quantize
    v, m = sp.sp24_prune_compress(to_dev(Wf))
    q, s_w = synth.quantize_rows(sp.sp24_decompress(v, m, M, K).cpu().numpy())
    xq, s_x = synth.quantize_tensor(np.ascontiguousarray(d["X_f32"][:, :N]))
    scale = synth.dequant_scales(s_w, s_x)
    xt = np.ascontiguousarray(xq.T)
    step_bytes = M * K * 2 + K * N + 4 * M * N
    kernel_bytes = M * K * 5 // 8 + K * N + 4 * M * N + 4 * M
    copies = []
    for _ in range(n_copies(step_bytes, kernel_bytes)):
        vb, mb = sp.sp24_compressed_bytes(M, K, torch.int8)
        copies.append(dict(W=to_dev(q), X=to_dev(xt), scale=to_dev(scale),
                           vals=torch.empty(vb, dtype=torch.int8, device="cuda"),
                           meta=torch.empty(mb, dtype=torch.uint8, device="cuda"),
                           Y=torch.empty((N, M), dtype=torch.float32, device="cuda")))
    kernels = [Kernel("prune_compress_i8", lambda c: sp.sp24_prune_compress(c["W"], values=c["vals"], meta=c["meta"]),
                      M * K + M * K * 5 // 8, sources=("prune.hip", "sp24_device.h")),
               Kernel("gemm_i8", lambda c: sp.sp24_gemm_i8_ex(c["vals"], c["meta"], M, c["X"], scale=c["scale"],
                                                              layout="token", out=c["Y"]),
                      kernel_bytes, float(M) * N * K, "i8", ("gemm_i8_fewtok.hip", "sp24_device.h"))]

    def cpu_sample(budget_s):
        import oracle
        v8, m8 = oracle.prune_compress(q, oracle.I8)
        per = dict(prune_compress_i8=_fn_entry(_median_s(lambda: oracle.prune_compress(q, oracle.I8)), nbytes=M * K * 13 // 8),
                   decompress_i8=_fn_entry(_median_s(lambda: oracle.decompress(v8, m8, oracle.I8, M, K)), nbytes=M * K * 13 // 8))
        t, rows, extra = _gemm_rows_timed(lambda r: oracle.gemm_i8(v8, m8, xq, M, scale, rows=np.arange(r)), M,
                                          max(budget_s - per["prune_compress_i8"]["s"], 0.5), 64)
        per["gemm_i8"] = _fn_entry(t, flops=float(M) * N * K, extrapolated=extra, rows=rows, total_rows=M)
        return (per["prune_compress_i8"]["s"] + t,
                f"int8 prune/compress of the full {M}x{K} weight (median of 3) + GEMM on {rows} of {M} rows"
                + (", scaled to all rows" if extra else ""), per)

    cfg = dict(workload="llm_proj_11008x4096_int8", M=M, K=K, N=N,
               weight="fp32 N(0,0.02^2) seed 37, 2:4 magnitude, per-row int8 at 99.99 % coverage",
               activations=f"fp32 N(0,1) seed 38, first {N} columns, per-tensor int8 at 99.99 % coverage",
               out="fp32 (int32 accumulate, per-channel dequant)", step="prune_compress int8 + gemm_i8",
               layout="token-major: X N x K, Y N x M")
    return dict(name=f"llm_proj_11008x4096_int8_n{N}", dtype="i8", unit="TOP/s", config=cfg,
                flops=2.0 * M * N * K, copies=copies, kernels=kernels, dense_ref=None, cpu_sample=cpu_sample)


WORKLOADS = {"vit_b16_fc1": workload_vit, "single_linear_256": workload_single, "bert_ffn_int8": workload_bert_int8,
             "bert_ffn_int8_fused": workload_bert_int8_fused,
             "llm_proj_11008x4096": workload_llm(11008), "llm_proj_4096x4096": workload_llm(4096),
             "ffn_28672x8192": workload_ffn, "llm_proj_11008x4096_int8": workload_llm_int8}


# ----------------------------------------------------------------------------- HBM traffic

def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, k: Kernel):
    """HBM bytes per launch of kernel k from the committed counter summary (FETCH_SIZE + WRITE_SIZE, each
    scaled by a plain copy's reading), or None when there is none or the kernel's source has changed
    since the counters were taken."""
    path = os.path.join(PROFILES, f"{k.name}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, v = line.split(":", 1)
            kv[key.strip()] = v.strip()
    if kv.get("kernel_source_digest") != source_digest(k.sources):
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def copy_calibration(mib: int, reps: int):
    """A plain device-to-device copy of a known size, for scaling FETCH_SIZE / WRITE_SIZE readings."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes_read=n, copy_bytes_written=n, reps=reps)), flush=True)


# ----------------------------------------------------------------------------- timing

def capture(calls):
    """One HIP graph holding the given calls in order (captured on torch's capture stream, which the
    library launches on), so the timed region runs them back to back without host gaps."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    return g


def kernel_time_ms(fn, copies, steps, warmup):
    """Average duration of fn(copy) over `steps` launches rotating the copies: the launches are replayed
    from one HIP graph bracketed by HIP events on the stream they run on."""
    nc = len(copies)
    for i in range(warmup):
        fn(copies[i % nc])
    torch.cuda.synchronize()
    g = capture([lambda i=i: fn(copies[i % nc]) for i in range(steps)])
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def launch_stats_us(fn, copies, steps):
    """Per-launch durations of fn(copy) from a pair of HIP events around each launch (rotating copies):
    the launches are queued behind a spin kernel on the same stream, so the GPU runs them back to back
    while the host enqueues; returns (median, p10, p90) in microseconds."""
    nc = len(copies)
    fn(copies[0])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    try:
        torch.cuda._sleep(int(4e7 + steps * 4e5))  # about 20 ms + 0.2 ms per launch at 2 GHz
    except Exception:
        pass
    for i in range(steps):
        ev[i][0].record()
        fn(copies[i % nc])
        ev[i][1].record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


def stream_floor_us(nbytes: int, steps: int):
    """The achievable floor for a kernel that must read nbytes once: a plain streaming read of exactly that many
    bytes (sp24_bench_stream_read), rotated over enough buffer copies that the launches cycle over more than
    twice the Infinity Cache, as the kernels are. Returns (average us, copies)."""
    nb = (int(nbytes) + 15) // 16 * 16
    n = max(2, min(64, int(np.ceil(2 * CACHE_BYTES / nb)) + 1))
    bufs = [dict(src=torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)) for _ in range(n)]
    sink = sp.sp24_bench_stream_read(bufs[0]["src"])
    t = kernel_time_ms(lambda c: sp.sp24_bench_stream_read(c["src"], nb, sink), bufs, steps, 2) * 1e3
    del bufs
    torch.cuda.empty_cache()
    return t, n


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_steps(w, steps, warmup):
    """Whole steps: W eager warmup steps, then exactly K steps replayed from one HIP graph, timed with the
    host clock between two synchronizations. Per kernel: `kernel_time_ms` for each kernel of the step."""
    copies, kernels = w["copies"], w["kernels"]

    def step(c):
        for k in kernels:
            k.fn(c)

    nc = len(copies)
    for i in range(warmup):
        step(copies[i % nc])
    torch.cuda.synchronize()
    g = capture([lambda i=i: step(copies[i % nc]) for i in range(steps)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    per_kernel_ms = {k.name: kernel_time_ms(k.fn, copies, steps, 1) for k in kernels}
    return t_total, per_kernel_ms


def roofline(k: Kernel, t_s: float, workload: str):
    gbs = k.nbytes / t_s / 1e9
    peak_tf = DENSE_PEAK[k.dtype]
    tf = k.flops / t_s / 1e12
    t_hbm = k.nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = k.flops / (peak_tf * 1e12)
    t_alu = k.valu_slots / (VALU_PEAK_TSLOTS * 1e12)
    if t_alu > max(t_hbm, t_mfma):
        ts = k.valu_slots / t_s / 1e12
        r = dict(bound="alu", achieved=round(ts, 2), peak=round(VALU_PEAK_TSLOTS, 2), unit="Tslot/s",
                 frac=round(ts / VALU_PEAK_TSLOTS, 4))
    elif k.flops == 0 or t_hbm >= t_mfma:
        r = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        r = dict(bound="mfma", achieved=round(tf, 1), peak=peak_tf, unit="TOP/s" if k.dtype == "i8" else "TFLOP/s",
                 frac=round(tf / peak_tf, 4))
    r["traffic"] = measured_traffic(workload, k)
    r["kernel"] = k.name
    r["algorithmic_bytes"] = int(k.nbytes)
    if k.flops:
        r["algorithmic_flops"] = k.flops
        r["mfma_frac"] = round(tf / peak_tf, 4)
    r["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    if k.valu_slots:
        r["valu_slots"] = k.valu_slots
        r["alu_frac"] = round(k.valu_slots / t_s / 1e12 / VALU_PEAK_TSLOTS, 4)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ffn_28672x8192", choices=sorted(WORKLOADS))
    ap.add_argument("--n", type=int, default=0, help="tokens N for the llm_proj_* and ffn_* workloads (ffn default 8192)")
    ap.add_argument("--layout", default="token", choices=("token", "feature"),
                    help="activations token-major (X N x K, Y N x M, a Linear layer's layout) or feature-major")
    ap.add_argument("--shard-m", type=int, default=1, metavar="G",
                    help="ffn_* / llm_proj_* (bf16): time one GPU's share of the layer split by output channels over G "
                         "GPUs (rows [0, M/G)); the other GPUs' shares are the same kernel on other rows")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-ref", action="store_true", help="skip timing the dense bf16 GEMM of the same shape")
    ap.add_argument("--no-sclk-probe", action="store_true", help="skip the shader-clock probe (sp24_probe_sclk)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (to scale FETCH_SIZE / WRITE_SIZE counter readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards with no "
              "communication: by tokens or by output channels)", file=sys.stderr)
        sys.exit(2)
    if args.shard_m < 1 or (args.shard_m > 1 and not (args.workload.startswith("ffn_") or
                                                       args.workload in ("llm_proj_11008x4096", "llm_proj_4096x4096"))):
        print("--shard-m applies to the bf16 ffn_* and llm_proj_* workloads, with G >= 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return
    sp.load_library()
    w = WORKLOADS[args.workload](args)
    t_total, per_kernel_ms = timed_steps(w, args.steps, args.warmup)
    ms_per_step = 1e3 * t_total / args.steps
    value = w["flops"] / (ms_per_step * 1e-3) / 1e12

    by_name = {k.name: k for k in w["kernels"]}
    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    roof = roofline(by_name[dom], per_kernel_ms[dom] * 1e-3, w["name"])
    kernels = {}
    for k in w["kernels"]:
        t = per_kernel_ms[k.name] * 1e-3
        e = dict(avg_us=round(t * 1e6, 2), gbs_algorithmic=round(k.nbytes / t / 1e9, 1))
        if k.flops:
            e["tflops_dense_equiv"] = round(2 * k.flops / t / 1e12, 1)
        # per-launch spread (HIP events around each launch, rotated copies: caches flushed by the rotation)
        med, p10, p90 = launch_stats_us(k.fn, w["copies"], args.steps)
        e.update(median_us=round(med, 2), p10_us=round(p10, 2), p90_us=round(p90, 2))
        # warm: the same launch repeated on one copy, so whatever fits stays in the caches (labelled as such)
        e["warm_avg_us"] = round(kernel_time_ms(k.fn, w["copies"][:1], args.steps, 1) * 1e3, 2)
        kernels[k.name] = e
    # GEMMs that stream their weight (few tokens: at most 64 flop per byte, reads dominate) and the column
    # norms (a pure read of X): the measured streaming-read floor of the same bytes beside the spec peak
    for k in w["kernels"]:
        if (k.flops and k.flops / k.nbytes <= 64) or k.name == "col_norms":
            f_us, n = stream_floor_us(k.nbytes, args.steps)
            e = kernels[k.name]
            e.update(floor_us=round(f_us, 2), floor_gbs=round(k.nbytes / f_us / 1e3, 1),
                     frac_of_floor=round(f_us / e["avg_us"], 4), hbm_frac=round(k.nbytes / e["avg_us"] / 1e3 / HBM_PEAK_GBS, 4))
            if k.name == dom:
                roof.update(floor_us=e["floor_us"], floor_gbs=e["floor_gbs"], frac_of_floor=e["frac_of_floor"])
    roof["median_us"] = kernels[dom]["median_us"]
    roof["p10_us"], roof["p90_us"] = kernels[dom]["p10_us"], kernels[dom]["p90_us"]

    if not args.no_sclk_probe:
        # the shader clock under sustained matrix-core load: the MFMA peak above assumes 2.4 GHz
        pr = sp.sp24_probe_sclk(iters=16000)
        roof["sclk_mhz"] = round(pr["sclk_mhz"], 1)
        roof["cycles_per_smfmac"] = round(pr["cycles_per_smfmac"], 2)
        k = by_name[dom]
        if k.flops:
            peak_sclk = DENSE_PEAK[k.dtype] * pr["sclk_mhz"] / SPEC_SCLK_MHZ
            roof["mfma_peak_at_sclk"] = round(peak_sclk, 1)
            roof["mfma_frac_at_sclk"] = round(k.flops / (per_kernel_ms[dom] * 1e-3) / 1e12 / peak_sclk, 4)

    if not args.no_dense_ref and w.get("dense_ref"):
        for name, fn in w["dense_ref"]().items():
            t_dense = kernel_time_ms(fn, w["copies"], args.steps, args.warmup)
            kernels[name] = dict(avg_us=round(t_dense * 1e3, 2))
            key = "speedup_vs_dense" if name == "dense_bf16_matmul_same_shape" else "speedup_vs_dense_same_tiling"
            kernels["gemm_bf16"][key] = round(t_dense / per_kernel_ms["gemm_bf16"], 3)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        t_cpu, sample, per_fn = w["cpu_sample"](args.cpu_budget)
        cores = oracle.threads()
        cpu = dict(value=round(w["flops"] / t_cpu / 1e12, 6), unit=w["unit"], cores=cores, cpu_model=cpu_model(),
                   kind="oracle", sample=sample, est_s_per_step=round(t_cpu, 3),
                   extrapolated=any("extrapolated" in e for e in per_fn.values()), per_function=per_fn)

    out = dict(metric="2:4 sparse GEMM dense-equiv TFLOP/s + % sparse-MFMA peak; prune GB/s", value=round(value, 2),
               unit=w["unit"], n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_per_step, 4),
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype=w["dtype"],
               data="synthetic (seeded numpy draws shaped like the workload; no dataset or checkpoint)",
               config=w["config"], roofline=roof, cpu_baseline=cpu, kernels=kernels,
               buffer_copies=len(w["copies"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
