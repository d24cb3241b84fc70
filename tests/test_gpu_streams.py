"""Streams and HIP graphs. The library keeps no per-call state and allocates nothing, so calls on different
streams are independent and a captured sequence of calls replays the same kernels on whatever the captured
buffers hold. Both are checked here against the same calls made eagerly, one after another, on the default
stream: results must be bit-identical (the same kernels run on the same inputs).

The path under test is the whole one: column norms, Wanda and magnitude prune/compress, the bf16 GEMM through
its tiled, few-token and skinny kernels, and the fused int8 GEMM (bias, GELU, int8 codes) through its tiled and
few-token kernels. Graph replays are checked over several rounds, with new inputs copied into the captured
buffers and eager work and synchronizations between the replays.
"""
import numpy as np
import pytest
import torch

import structured_sparse_gemm_sp24_amd as sp
from structured_sparse_gemm_sp24_amd import synth
from tests.gpu_util import dev, require_gpu, say

pytestmark = pytest.mark.gpu

M, K = 1024, 2048          # bf16 weight
M8, K8 = 768, 1024         # int8 weight
NCAL = 256                 # calibration tokens for the Wanda norms
# (tokens, layout) of the bf16 products: tiled token-major, few-token token-major, skinny feature-major
BF16_CASES = ((200, "token"), (8, "token"), (40, "feature"))
# tokens of the int8 products (token-major): tiled and few-token
I8_CASES = (300, 16)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(seed):
    """One seeded set of host inputs for the whole path."""
    rng = np.random.default_rng(seed)
    d = dict(
        W=synth.normal_bf16(seed + 1, (M, K), 0.02),
        Xcal=synth.heavy_tailed_bf16(seed + 2, K, NCAL),
        X={n: synth.normal_bf16(seed + 3 + n, (n, K) if lay == "token" else (K, n)) for n, lay in BF16_CASES},
        W8=rng.integers(-128, 128, size=(M8, K8), dtype=np.int8),
        X8={n: rng.integers(-128, 128, size=(n, K8), dtype=np.int8) for n in I8_CASES},
        scale=(rng.random(M8) * 1e-3 + 1e-4).astype(np.float32),
        bias=(rng.standard_normal(M8) * 0.02).astype(np.float32),
    )
    return d


def _to_dev(h):
    return dict(W=dev(h["W"], "bf16"), Xcal=dev(h["Xcal"], "bf16"), X={n: dev(x, "bf16") for n, x in h["X"].items()},
                W8=dev(h["W8"]), X8={n: dev(x) for n, x in h["X8"].items()}, scale=dev(h["scale"]),
                bias=dev(h["bias"]))


def _outputs(d):
    """Preallocated outputs for one pass (so a captured pass allocates nothing)."""
    vb, mb = sp.sp24_compressed_bytes(M, K, torch.bfloat16)
    vb8, mb8 = sp.sp24_compressed_bytes(M8, K8, torch.int8)
    out = dict(norms=torch.empty(K, dtype=torch.float32, device="cuda"),
               v_w=torch.empty(vb // 2, dtype=torch.bfloat16, device="cuda"),
               m_w=torch.empty(mb, dtype=torch.uint8, device="cuda"),
               v_m=torch.empty(vb // 2, dtype=torch.bfloat16, device="cuda"),
               m_m=torch.empty(mb, dtype=torch.uint8, device="cuda"),
               v8=torch.empty(vb8, dtype=torch.int8, device="cuda"),
               m8=torch.empty(mb8, dtype=torch.uint8, device="cuda"))
    for n, lay in BF16_CASES:
        out[f"Y{n}"] = torch.empty((n, M) if lay == "token" else (M, n), dtype=torch.bfloat16, device="cuda")
    for n in I8_CASES:
        out[f"H{n}"] = torch.empty((n, M8), dtype=torch.int8, device="cuda")
    return out


def _pass(d, o):
    """The whole path on the current stream: Wanda chain, magnitude prune, bf16 and fused int8 GEMMs."""
    sp.sp24_col_norms(d["Xcal"], norms=o["norms"])
    sp.sp24_prune_compress(d["W"], score=sp.SP24_SCORE_WANDA, norms=o["norms"], values=o["v_w"], meta=o["m_w"])
    sp.sp24_prune_compress(d["W"], values=o["v_m"], meta=o["m_m"])
    for n, lay in BF16_CASES:
        sp.sp24_gemm_bf16_ex(o["v_w"], o["m_w"], M, d["X"][n], layout=lay, out=o[f"Y{n}"])
    sp.sp24_prune_compress(d["W8"], values=o["v8"], meta=o["m8"])
    for n in I8_CASES:
        sp.sp24_gemm_i8_fused(o["v8"], o["m8"], M8, d["X8"][n], d["scale"], bias=d["bias"], activation="gelu",
                              out_dtype=torch.int8, out_scale=0.02, layout="token", out=o[f"H{n}"])


def _bytes(t):
    return t.contiguous().view(-1).view(torch.uint8)


def _same(a, b):
    """Every output of two passes, bit for bit; returns the names that differ."""
    return [k for k in a if not torch.equal(_bytes(a[k]), _bytes(b[k]))]


def test_concurrent_streams_equal_sequential():
    """Four streams, each running the whole path on its own inputs at the same time, against the same passes
    run one after another on the default stream."""
    seeds = (101, 202, 303, 404)
    ins = [_to_dev(_inputs(s)) for s in seeds]
    say("streams: sequential reference passes on the default stream")
    ref = []
    for d in ins:
        o = _outputs(d)
        _pass(d, o)
        ref.append(o)
    torch.cuda.synchronize()
    say("streams: four concurrent streams")
    outs = [_outputs(d) for d in ins]
    main = torch.cuda.current_stream()
    streams = [torch.cuda.Stream() for _ in seeds]  # default priority
    for s in streams:
        s.wait_stream(main)  # inputs and outputs were made on the default stream
    for _ in range(2):  # two rounds, so that passes of different streams overlap in time
        for s, d, o in zip(streams, ins, outs):
            with torch.cuda.stream(s):
                _pass(d, o)
    torch.cuda.synchronize()
    for i, (o, r) in enumerate(zip(outs, ref)):
        assert not _same(o, r), (seeds[i], _same(o, r))
    # the passes really differ from stream to stream (distinct inputs, distinct outputs)
    assert not torch.equal(_bytes(outs[0]["Y200"]), _bytes(outs[1]["Y200"]))


def test_graph_replays_equal_eager():
    """The whole path captured once in a HIP graph, replayed over three rounds of new inputs copied into the
    captured buffers, each replay against an eager pass over the same inputs."""
    static = _to_dev(_inputs(500))
    o_graph = _outputs(static)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _pass(static, o_graph)  # eager warm-up before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph: capture of the whole path")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _pass(static, o_graph)
    torch.cuda.synchronize()
    for rnd, seed in enumerate((600, 700, 800)):
        say(f"graph: replay {rnd} with inputs of seed {seed}")
        h = _inputs(seed)
        fresh = _to_dev(h)
        # new inputs into the captured buffers (copies are eager work between the replays)
        static["W"].copy_(fresh["W"])
        static["Xcal"].copy_(fresh["Xcal"])
        static["W8"].copy_(fresh["W8"])
        static["scale"].copy_(fresh["scale"])
        static["bias"].copy_(fresh["bias"])
        for n in static["X"]:
            static["X"][n].copy_(fresh["X"][n])
        for n in static["X8"]:
            static["X8"][n].copy_(fresh["X8"][n])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_eager = _outputs(fresh)
        _pass(fresh, o_eager)
        torch.cuda.synchronize()
        diff = _same(o_graph, o_eager)
        assert not diff, (rnd, diff)
        # and a second replay on the same inputs gives the same bits again
        g.replay()
        torch.cuda.synchronize()
        assert not _same(o_graph, o_eager), rnd
