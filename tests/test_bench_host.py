"""Host checks of bench.py's roofline choice (no GPU: the function only prices given bytes, flops and slots)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _k(nbytes, flops, dtype="bf16", slots=0.0):
    return bench.Kernel("k", None, nbytes, flops, dtype, (), valu_slots=slots)


def test_roofline_picks_the_binding_roof():
    # 28672 x 8192 x 8192 bf16: MFMA-bound; 1550 us is 49.3 % of the dense bf16 peak
    M, K, N = 28672, 8192, 8192
    r = bench.roofline(_k(M * K * 9 // 8 + 2 * K * N + 2 * M * N, float(M) * N * K), 1550e-6, "none")
    assert r["bound"] == "mfma" and abs(r["frac"] - M * N * K / 1550e-6 / 2516.6e12) < 1e-4
    # 11008 x 4096 at N = 16: HBM-bound
    M, K, N = 11008, 4096, 16
    r = bench.roofline(_k(M * K * 9 // 8 + 2 * K * N + 2 * M * N, float(M) * N * K), 13e-6, "none")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    # the fused int8 epilogue with GELU: VALU slots outweigh bytes and flops
    M, K, N = 3072, 768, 8192
    slots = float(bench.GELU_I8_SLOTS_PER_OUTPUT) * M * N
    r = bench.roofline(_k(M * K * 5 // 8 + K * N + M * N + 8 * M, float(M) * N * K, "i8", slots), 33.2e-6, "none")
    assert r["bound"] == "alu" and r["unit"] == "Tslot/s"
    assert abs(bench.VALU_PEAK_TSLOTS - 39.3216) < 1e-6
    assert abs(r["frac"] - slots / 33.2e-6 / 1e12 / bench.VALU_PEAK_TSLOTS) < 1e-4


def test_buffer_rotation_covers_the_infinity_cache():
    MB = 1 << 20
    # the FFN step (about 1.34 GB) rotates three copies; a 51 MB kernel cycles over more than 512 MB
    assert bench.n_copies(1340 * MB, 868 * MB) == 3
    n = bench.n_copies(60 * MB, 51 * MB)
    assert n * 51 * MB > 2 * bench.CACHE_BYTES and n <= 64
    # never fewer than three, whatever the budget
    assert bench.n_copies(10 << 30, 5 << 30) == 3


def test_shard_rows_takes_one_gpus_share():
    import argparse
    import numpy as np
    W = np.arange(28672 * 4, dtype=np.uint16).reshape(28672, 4)
    Ws, cfg, name = bench.shard_rows(W, argparse.Namespace(shard_m=8), dict(M=28672), "ffn")
    assert Ws.shape == (3584, 4) and np.array_equal(Ws, W[:3584]) and cfg["M"] == 3584 and name == "ffn_mshard8"
    # shares round up to whole 16-row blocks; G = 1 is the whole layer
    Ws, cfg, _ = bench.shard_rows(W[:11008], argparse.Namespace(shard_m=3), dict(M=11008), "llm")
    assert Ws.shape[0] == 3680 and 3 * 3680 >= 11008
    assert bench.shard_rows(W, argparse.Namespace(shard_m=1), {}, "x")[0] is W
