"""Benchmark of the 2:4 sparse hot path on one MI355X.

One step = one pass of the workload's whole path over its synthetic batch, e.g. for the default
ViT-B/16 MLP fc1 workload: 2:4 magnitude prune + compress of W (3072 x 768 bf16), then the sparse
GEMM Y = W_2:4 . X (X 768 x 6304 bf16, Y bf16). Inputs are resident in HBM before timing; steps
rotate over enough copies of every buffer (> 2x the 256 MB Infinity Cache) that each step reads its
operands from HBM, not from cache.

Prints ONE JSON line: dense-equivalent TFLOP/s of the step (2*M*N*K per step), the dominant
kernel's roofline (its own average duration from HIP events on the launch stream, algorithmic bytes
or flops per launch), and the CPU oracle timed on a bounded sample of the same workload.
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
SPARSE_BF16_PEAK_TF = 5033.2   # dense-equivalent, 2:4 sparse MFMA
SPARSE_I8_PEAK_TOPS = 10066.4
DENSE_BF16_PEAK_TF = 2516.6
CACHE_BYTES = 256 << 20        # MI355X Infinity Cache
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "structured_sparse_gemm_sp24_amd", "csrc")


def to_dev(a, kind=None):
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def n_copies(step_bytes: int) -> int:
    return max(1, min(64, int(np.ceil(2 * CACHE_BYTES / max(step_bytes, 1)))))


# ----------------------------------------------------------------------------- workloads
# Each builder returns a dict with: name, config, flops (dense-equivalent per step), copies (list of
# per-copy buffer dicts), step(c) (runs one pass on copy c), gemm(c) (the dominant kernel alone),
# gemm_bytes / gemm_flops (algorithmic, per launch), bound, dtype, cpu_sample() (oracle timing).

def workload_vit(args):
    d = synth.vit_b16_fc1()
    M, K = d["W_bf16"].shape
    N = d["X_bf16"].shape[1]
    step_bytes = M * K * 2 + M * K * 9 // 8 + K * N * 2 + M * N * 2
    copies = []
    for _ in range(n_copies(step_bytes)):
        W = to_dev(d["W_bf16"], "bf16")
        vb, mb = sp.sp24_compressed_bytes(M, K, torch.bfloat16)
        copies.append(dict(W=W, X=to_dev(d["X_bf16"], "bf16"),
                           vals=torch.empty(vb // 2, dtype=torch.bfloat16, device="cuda"),
                           meta=torch.empty(mb, dtype=torch.uint8, device="cuda"),
                           Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))

    def prune(c):
        sp.sp24_prune_compress(c["W"], values=c["vals"], meta=c["meta"])

    def gemm(c):
        sp.sp24_gemm_bf16(c["vals"], c["meta"], M, c["X"], out=c["Y"])

    def dense_ref():
        # dense bf16 GEMM of the same shape (torch.matmul -> hipBLASLt) on the decompressed pruned weight
        c0 = copies[0]
        sp.sp24_prune_compress(c0["W"], values=c0["vals"], meta=c0["meta"])
        Wd = sp.sp24_decompress(c0["vals"], c0["meta"], M, K)
        return [(lambda c, Wd=Wd: torch.matmul(Wd, c["X"], out=c["Y"]))]

    def cpu_sample(budget_s):
        import oracle
        t0 = time.perf_counter()
        v, m = oracle.prune_compress(d["W_bf16"], oracle.BF16)
        t_prune = time.perf_counter() - t0
        rows = 8
        t0 = time.perf_counter()
        oracle.gemm_bf16(v, m, d["X_bf16"], M, rows=np.arange(rows))
        t_small = time.perf_counter() - t0
        rows = int(min(M, max(8, rows * (budget_s - t_prune) / max(t_small, 1e-6))))
        t0 = time.perf_counter()
        oracle.gemm_bf16(v, m, d["X_bf16"], M, rows=np.arange(rows))
        t_rows = time.perf_counter() - t0
        t_step = t_prune + t_rows * M / rows
        return t_step, f"prune/compress of the full {M}x{K} W + GEMM on {rows} of {M} rows, scaled to all rows"

    return dict(name="vit_b16_fc1", dtype="bf16",
                config=dict(workload="vit_b16_fc1", M=M, K=K, N=N, weight="bf16 N(0,0.02^2) seed 11",
                            activations="bf16 N(0,1) seed 12, N = 32 images x 197 tokens", score="magnitude",
                            out="bf16", step="prune_compress + gemm_bf16"),
                flops=2.0 * M * N * K, copies=copies, kernels=dict(prune_compress=prune, gemm_bf16=gemm),
                dominant="gemm_bf16", sources=("gemm_bf16_tiled.hip", "sp24_device.h"),
                dense_ref=dense_ref, gemm_bytes=M * K * 9 // 8 + K * N * 2 + M * N * 2, gemm_flops=2.0 * M * N * K,
                prune_bytes=M * K * 2 + M * K * 9 // 8, cpu_sample=cpu_sample, unit="TFLOP/s")


WORKLOADS = {"vit_b16_fc1": workload_vit}


# ----------------------------------------------------------------------------- HBM traffic

def source_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(w):
    """HBM bytes per launch of the dominant kernel from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy's reading), or None when there is none or the kernel's source
    has changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{w['dominant']}_{w['name']}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != source_digest(w["sources"]):
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

def kernel_time_ms(fn, copies, steps, warmup):
    """Average duration of fn(copy) from HIP events recorded on the launch stream, rotating copies."""
    nc = len(copies)
    for i in range(warmup):
        fn(copies[i % nc])
    ev = []
    for i in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(copies[i % nc])
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def timed_steps(w, steps, warmup):
    copies, kernels = w["copies"], w["kernels"]
    names = list(kernels)

    def step(c):
        for n in names:
            kernels[n](c)

    nc = len(copies)
    for i in range(warmup):
        step(copies[i % nc])
    torch.cuda.synchronize()
    # whole steps, host clock around K steps bracketed by synchronizations
    t0 = time.perf_counter()
    for i in range(steps):
        step(copies[i % nc])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t0
    # per-kernel durations: HIP events on the launch stream around each kernel, same rotation
    ev = {n: [] for n in names}
    for i in range(steps):
        c = copies[i % nc]
        for n in names:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            kernels[n](c)
            e1.record()
            ev[n].append((e0, e1))
    torch.cuda.synchronize()
    per_kernel_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}
    return t_total, per_kernel_ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="vit_b16_fc1", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-ref", action="store_true", help="skip timing the dense bf16 GEMM of the same shape")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (to scale FETCH_SIZE / WRITE_SIZE counter readings)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path shards with no "
              "communication: by tokens or by output channels, see DESIGN.md)", file=sys.stderr)
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

    dom = w["dominant"]
    t_dom = per_kernel_ms[dom] * 1e-3
    achieved_gbs = w["gemm_bytes"] / t_dom / 1e9
    achieved_tf = w["gemm_flops"] / t_dom / 1e12
    peak_tf = SPARSE_I8_PEAK_TOPS if w["dtype"] == "i8" else SPARSE_BF16_PEAK_TF
    ideal_hbm = w["gemm_bytes"] / (HBM_PEAK_GBS * 1e9)
    ideal_mfma = w["gemm_flops"] / (peak_tf * 1e12)
    if ideal_hbm >= ideal_mfma:
        roof = dict(bound="hbm", achieved=round(achieved_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved_gbs / HBM_PEAK_GBS, 4), traffic=measured_traffic(w))
    else:
        roof = dict(bound="mfma", achieved=round(achieved_tf, 1), peak=peak_tf,
                    unit="TOP/s" if w["dtype"] == "i8" else "TFLOP/s", frac=round(achieved_tf / peak_tf, 4),
                    traffic=measured_traffic(w))
    roof["algorithmic_bytes"] = w["gemm_bytes"]
    roof["kernel"] = dom
    roof["mfma_frac"] = round(achieved_tf / peak_tf, 4)
    roof["hbm_frac"] = round(achieved_gbs / HBM_PEAK_GBS, 4)

    kernels = {}
    for n, ms in per_kernel_ms.items():
        kernels[n] = dict(avg_us=round(ms * 1e3, 2))
    kernels[dom]["tflops_dense_equiv"] = round(achieved_tf, 1)
    kernels[dom]["gbs_algorithmic"] = round(achieved_gbs, 1)
    if "prune_compress" in per_kernel_ms:
        kernels["prune_compress"]["gbs_algorithmic"] = round(w["prune_bytes"] / (per_kernel_ms["prune_compress"] * 1e-3)
                                                            / 1e9, 1)

    if not args.no_dense_ref and w.get("dense_ref"):
        fns = w["dense_ref"]()
        t_dense = sum(kernel_time_ms(f, w["copies"], args.steps, args.warmup) for f in fns)
        kernels["dense_bf16_matmul_same_shape"] = dict(avg_us=round(t_dense * 1e3, 2))
        kernels[dom]["speedup_vs_dense"] = round(t_dense / per_kernel_ms[dom], 3)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        t_cpu, sample = w["cpu_sample"](args.cpu_budget)
        cores = len(os.sched_getaffinity(0))
        cpu = dict(value=round(w["flops"] / t_cpu / 1e12, 6), unit=w["unit"], cores=cores, kind="oracle",
                   sample=sample, est_s_per_step=round(t_cpu, 3))

    out = dict(metric="2:4 sparse GEMM dense-equiv TFLOP/s + % sparse-MFMA peak; prune GB/s", value=round(value, 2),
               unit=w["unit"], n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_per_step, 4),
               higher_is_better=True, scaling="weak", vs_baseline=None, dtype=w["dtype"],
               data="synthetic (seeded numpy draws shaped like the workload; no dataset or checkpoint)",
               config=w["config"], roofline=roof, cpu_baseline=cpu, kernels=kernels,
               buffer_copies=len(w["copies"]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
