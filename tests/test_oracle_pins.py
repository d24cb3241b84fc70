"""Pins for the CPU oracle: each test ties it to something other than itself -- the pages' worked
examples (tests/golden), brute force over every small case, closed forms, and library routines
(numpy/torch conversions and matmuls). These run without a GPU.

Where a test needs a second statement of the selection rule, it uses a different algorithm from the
oracle's (the oracle counts how many elements beat each one; the tests sort, or enumerate pairs).
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from structured_sparse_gemm_sp24_amd import synth
from tests.conftest import read_golden
from tests.layout_ref import padding_ok, to_row_major

ESIZE = {oracle.BF16: 2, oracle.FP16: 2, oracle.FP32: 4, oracle.I8: 1}


def compress_rm(W, dt, score=oracle.MAGNITUDE, norms=None, val_dtype=None):
    """Oracle compression viewed row-major: (values M x K/2, meta M x K/8, flat values, flat meta)."""
    vdt = dt if val_dtype is None else val_dtype
    v, m = oracle.prune_compress(W, dt, score, norms, val_dtype)
    M, K = W.shape
    assert padding_ok(v, m, M, K, ESIZE[vdt])
    vr, mr = to_row_major(v, m, M, K, ESIZE[vdt])
    return vr, mr, v, m

# ----------------------------------------------------------------- independent helpers


def top2_by_sort(scores: np.ndarray) -> np.ndarray:
    """Kept positions (ascending) of each group of 4 along the last axis: stable sort by descending
    score, so equal scores keep their index order and the lower index wins."""
    s = scores.reshape(-1, 4)
    order = np.argsort(-s, axis=1, kind="stable")[:, :2]
    return np.sort(order, axis=1)


def top2_by_pairs(scores4) -> tuple:
    """Of the six pairs, the one whose sorted score pair is largest; among equal ones the
    lexicographically smallest index pair."""
    best = None
    for a, b in itertools.combinations(range(4), 2):
        key = tuple(sorted((scores4[a], scores4[b]), reverse=True))
        if best is None or key > best[0]:
            best = (key, (a, b))
    return best[1]


def meta_nibbles(meta: np.ndarray, K: int) -> np.ndarray:
    m = np.asarray(meta, np.uint8)
    lo, hi = m & 0xF, m >> 4
    return np.stack([lo, hi], axis=-1).reshape(m.shape[0], K // 4)


def dense_from_positions(Wd: np.ndarray, pos: np.ndarray) -> np.ndarray:
    M, K = Wd.shape
    out = np.zeros_like(Wd)
    g = np.arange(K // 4)
    for t in range(2):
        cols = 4 * g[None, :] + pos.reshape(M, K // 4, 2)[:, :, t]
        np.put_along_axis(out, cols, np.take_along_axis(Wd, cols, axis=1), axis=1)
    return out


def f16_bits(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


# ----------------------------------------------------------------- worked examples from the pages


def test_orin7_q1_exercise_fp16():
    g = read_golden("orin7_q1_exercise.txt")
    w = np.array([float(x) for x in g["weights"].split()])
    # the page's slice is 8 weights; the library works on rows of a multiple of 16, so the slice is
    # followed by 8 zero weights (their group picks positions 0 and 1, values +0)
    W = np.concatenate([f16_bits(w), np.zeros(8, np.uint16)]).reshape(1, 16)
    vals, meta, _, _ = compress_rm(W, oracle.FP16)
    assert [f"{v:04X}" for v in vals[0, :4]] == g["values_fp16_hex"].split()
    assert meta[0, 0] == int(g["meta_hex"], 16)
    pruned = np.array([float(x) for x in g["pruned"].split()])
    dense = oracle.decompress(*oracle.prune_compress(W, oracle.FP16), oracle.FP16, 1, 16)
    assert np.array_equal(dense[0, :8], f16_bits(pruned))
    # storage of the slice: every kept value is 16 bits, every group 4 bits of metadata
    stored = vals[0, :4].size * 16 + 1 * 8
    assert stored == int(g["stored_bits"]) and w.size * 16 == int(g["dense_bits"])
    pos = [tuple(int(c) for c in p.split(",")) for p in g["kept_positions"].split()]
    nib = meta_nibbles(meta, 16)[0, :2]
    assert [(n & 3, n >> 2) for n in nib] == pos


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP32])
def test_orin7_q1_exercise_other_dtypes(dt):
    g = read_golden("orin7_q1_exercise.txt")
    w = np.array([float(x) for x in g["weights"].split()] + [0] * 8, dtype=np.float32)
    W = synth.f32_to_bf16_bits(w).reshape(1, 16) if dt == oracle.BF16 else w.reshape(1, 16)
    _, meta, _, _ = compress_rm(W, dt)
    assert meta[0, 0] == int(g["meta_hex"], 16)


def test_orin7_hw_flow_encoding_and_gather():
    g = read_golden("orin7_hw_flow.txt")
    pre = np.array([float(x) for x in g["prepruned"].split()] + [0] * 12, dtype=np.float32)
    W = synth.f32_to_bf16_bits(pre).reshape(1, 16)
    vals, meta, vflat, mflat = compress_rm(W, oracle.BF16)
    page_vals = np.array([float(x) for x in g["values"].split()], dtype=np.float32)
    assert np.array_equal(vals[0, :2], synth.f32_to_bf16_bits(page_vals))  # the page's values, in bf16
    bits = g["meta_bits"].split()
    nib = meta_nibbles(meta, 16)[0, 0]
    assert (f"{nib & 3:02b}", f"{nib >> 2:02b}") == tuple(bits)
    assert nib == int(g["nibble_hex"], 16)
    # gather semantics: result = -0.5 * x1 + 0.2 * x3 for activations x0..x3
    x = np.array([float(v) for v in g["activations"].split()] + [1] * 12, dtype=np.float32)
    X = synth.f32_to_bf16_bits(x).reshape(16, 1)
    Y = oracle.gemm_bf16(vflat, mflat, X, 1)
    v = synth.bf16_bits_to_f32(vals[0, :2]).astype(np.float64)
    xs = synth.bf16_bits_to_f32(X[:, 0]).astype(np.float64)
    assert Y[0, 0] == v[0] * xs[1] + v[1] * xs[3]
    assert Y[0, 0] == pytest.approx(float(g["result"]), abs=11 * 2.0 ** -11)  # 0.2 rounded to bf16, times 11


def test_orin7_rule_beats_illustration():
    g = read_golden("orin7_hw_flow.txt")
    w = np.array([float(x) for x in g["rule_example"].split()] + [0] * 12, dtype=np.float32)
    vals, meta, _, _ = compress_rm(w.reshape(1, 16), oracle.FP32)
    nib = meta_nibbles(meta, 16)[0, 0]
    assert (nib & 3, nib >> 2) == tuple(int(c) for c in g["rule_kept_positions"].split(","))
    assert vals[0, :2].tolist() == [np.float32(float(x)) for x in g["rule_values"].split()]


# ----------------------------------------------------------------- brute force over small cases


def test_bruteforce_every_group_over_small_alphabet():
    """All 6^4 groups over {-2, -1, -0, +0, 1, 2}: the oracle's choice equals pair enumeration, kept
    values are bit copies (signed zero included) and pruned slots decompress to +0."""
    alphabet = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    groups = np.array(list(itertools.product(range(6), repeat=4)))
    W = alphabet[groups].reshape(1, -1)
    K = W.shape[1]
    vals, meta, vflat, mflat = compress_rm(W, oracle.FP32)
    nib = meta_nibbles(meta, K)[0]
    for gi, gidx in enumerate(groups):
        a, b = top2_by_pairs(np.abs(alphabet[gidx]).tolist())
        assert (nib[gi] & 3, nib[gi] >> 2) == (a, b), (gi, alphabet[gidx])
        assert vals[0, 2 * gi].view(np.uint32) == alphabet[gidx[a]].view(np.uint32)
        assert vals[0, 2 * gi + 1].view(np.uint32) == alphabet[gidx[b]].view(np.uint32)
    dense = oracle.decompress(vflat, mflat, oracle.FP32, 1, K)
    pos = np.array([[n & 3, n >> 2] for n in nib])
    ref = dense_from_positions(W, pos)
    assert np.array_equal(dense.view(np.uint32), ref.view(np.uint32))


def test_bruteforce_int8_heavy_ties():
    rng = np.random.default_rng(7)
    alphabet = np.array([-128, -127, -3, -1, 0, 1, 3, 127], dtype=np.int8)
    W = alphabet[rng.integers(0, len(alphabet), size=(64, 256))]
    vals, meta, vflat, mflat = compress_rm(W, oracle.I8)
    key = np.abs(W.astype(np.int32))  # |-128| = 128
    pos = top2_by_sort(key.reshape(64, -1))
    nib = meta_nibbles(meta, 256).reshape(-1)
    assert np.array_equal(nib & 3, pos[:, 0]) and np.array_equal(nib >> 2, pos[:, 1])
    assert np.array_equal(oracle.decompress(vflat, mflat, oracle.I8, 64, 256), dense_from_positions(W, pos))


# ----------------------------------------------------------------- k-of-4 masks


def topk_by_sort(scores: np.ndarray, k: int) -> np.ndarray:
    """Mask nibbles of each group of 4 along the last axis: the first k of a stable sort by descending
    score (equal scores keep index order, so the lower index wins)."""
    s = scores.reshape(-1, 4)
    order = np.argsort(-s, axis=1, kind="stable")[:, :k]
    return (1 << order).sum(axis=1)


def mask_nibbles(mask: np.ndarray, K: int) -> np.ndarray:
    m = np.asarray(mask, np.uint8)
    return np.stack([m & 0xF, m >> 4], axis=-1).reshape(m.shape[0], K // 4)


@pytest.mark.parametrize("keep", [1, 2, 3, 4])
def test_mask_bruteforce_every_group(keep):
    """All 6^4 groups over {-2, -1, -0, +0, 1, 2}: the k-of-4 mask equals a stable top-k sort, the
    masked weight keeps bit copies and writes +0 elsewhere."""
    alphabet = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    groups = np.array(list(itertools.product(range(6), repeat=4)))
    W = alphabet[groups].reshape(1, -1)
    K = W.shape[1]
    mask, out = oracle.prune_mask(W, oracle.FP32, keep)
    nib = mask_nibbles(mask, K)[0]
    assert np.array_equal(nib, topk_by_sort(np.abs(W), keep))
    bits = (nib[:, None] >> np.arange(4)[None, :]) & 1
    ref = np.where(bits.reshape(1, -1) == 1, W, np.float32(0.0))
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    assert np.all([bin(n).count("1") == keep for n in nib])


def test_mask_two_of_four_equals_compression_positions():
    for dt in (oracle.BF16, oracle.I8):
        W = (synth.normal_bf16(5, (37, 208)) if dt == oracle.BF16
             else np.random.default_rng(5).integers(-128, 128, size=(37, 208), dtype=np.int8))
        mask, _ = oracle.prune_mask(W, dt, 2)
        vals, meta, _, _ = compress_rm(W, dt)
        nib = meta_nibbles(meta, 208)
        assert np.array_equal(mask_nibbles(mask, 208), (1 << (nib & 3)) | (1 << (nib >> 2)))


@pytest.mark.parametrize("score", [oracle.MAGNITUDE, oracle.WANDA])
def test_progressive_masks_equal_direct(score):
    """NVIDIA blog, progressive sparse training (Figure 4): keep 3 of 4, then recompute on the remaining
    weights to keep 2 of 4. Without tuning in between, that equals the direct 2 of 4 mask (the dropped
    element scores 0 and stays last); so does every chain 4 -> 3 -> 2 -> 1."""
    W = synth.normal_bf16(9, (48, 256))
    W[:, ::7] = 0  # ties at zero
    norms = None
    if score == oracle.WANDA:
        norms = np.abs(np.random.default_rng(3).standard_normal(256)).astype(np.float32)
    cur = W
    for keep in (3, 2, 1):
        m_direct, out_direct = oracle.prune_mask(W, oracle.BF16, keep, score, norms)
        m_chain, out_chain = oracle.prune_mask(cur, oracle.BF16, keep, score, norms)
        assert np.array_equal(m_chain, m_direct), keep
        assert np.array_equal(out_chain, out_direct)
        cur = out_chain


# ----------------------------------------------------------------- channel permutation


def _golden_floats(g, key):
    return [float(x) for x in g[key].split()]


def test_permutation_golden_principle():
    g = read_golden("orin7_permutation.txt")
    row = np.array(_golden_floats(g, "row"), np.float32)
    W = np.tile(row, (3, 2))  # K is a multiple of 16: the 8-column row twice
    r0 = oracle.retained(W, oracle.FP32)
    perm = oracle.channel_permutation(W, oracle.FP32)
    r1 = oracle.retained(W, oracle.FP32, perm)
    f = float(np.float32(0.9)), float(np.float32(0.1))
    assert r0 == pytest.approx(6 * (3 * f[0] + f[1]), rel=1e-15)
    assert _golden_floats(g, "retained_before")[0] == pytest.approx(r0 / 6, rel=1e-6)
    assert r1 == pytest.approx(6 * 4 * f[0], rel=1e-15)
    assert _golden_floats(g, "retained_after")[0] == pytest.approx(r1 / 6, rel=1e-6)
    assert sorted(perm.tolist()) == list(range(16))
    # the page's one-group example keeps both large weights without any permutation
    ex = np.array(_golden_floats(g, "page_example_row"), np.float32).reshape(1, 4)
    pos = [int(x) for x in _golden_floats(g, "page_example_kept_positions")]
    W16 = np.tile(ex, (1, 4))
    vals, meta, _, _ = compress_rm(W16, oracle.FP32)
    nib = meta_nibbles(meta, 16)[0, 0]
    assert [nib & 3, nib >> 2] == pos


def test_permutation_two_groups_is_best_partition():
    """K = 8: one sweep is one round on the single pair, so the result must reach the best of all 35
    partitions of the 8 channels into two groups of four (enumerated independently here)."""
    rng = np.random.default_rng(21)
    for trial in range(20):
        W = rng.standard_normal((16, 8)).astype(np.float32)
        a = np.abs(W.astype(np.float64))
        best = -1.0
        for A in itertools.combinations(range(8), 4):
            B = [c for c in range(8) if c not in A]
            tA = np.sort(a[:, list(A)], axis=1)[:, -2:].sum(axis=1)
            tB = np.sort(a[:, B], axis=1)[:, -2:].sum(axis=1)
            best = max(best, float((tA + tB).sum()))
        perm = oracle.channel_permutation(W, oracle.FP32)
        assert sorted(perm.tolist()) == list(range(8))
        r = oracle.retained(W, oracle.FP32, perm)
        assert r == pytest.approx(best, rel=1e-12), trial


def test_permutation_schedule_meets_every_pair_once():
    """One sweep is G' - 1 rounds of G'/2 pairs (G' = G rounded up to even). Enumerated here from the
    oracle's own schedule: inside a round no group is in two pairs (the pairs of a round are
    independent), and over the sweep every two of the G groups meet exactly once, odd G included (the
    group drawn against the dummy sits the round out)."""
    for G in range(2, 41):
        Ge = G + (G & 1)
        seen = []
        for r in range(Ge - 1):
            pairs = [oracle.perm_pair(G, r, p) for p in range(Ge // 2)]
            pairs = [pr for pr in pairs if pr is not None]
            assert len(pairs) == G // 2, (G, r)  # every real group plays, except one when G is odd
            groups = [g for pr in pairs for g in pr]
            assert len(set(groups)) == len(groups), (G, r)
            assert all(0 <= a < b < G for a, b in pairs), (G, r)
            seen += pairs
        assert sorted(seen) == list(itertools.combinations(range(G), 2)), G


def _one_improvable_pair(G, a, b):
    """Two rows of 4G channels in which only groups a and b (a < b) can gain by re-partitioning:
    a = [9 9 9 0] keeps 18 of 27, b = [9 0 0 0] keeps 9; every other group is [20 20 0 0] and already
    keeps its two largest, and any pair that includes one of them holds at most four values that a
    split could keep, which it keeps already. The best split of (a, b) keeps 36."""
    W = np.tile(np.array([20, 20, 0, 0], np.float32), (2, G))
    W[:, 4 * a:4 * a + 4] = [9, 9, 9, 0]
    W[:, 4 * b:4 * b + 4] = [9, 0, 0, 0]
    W[1] = -W[1]  # the score is the magnitude
    return W


def test_permutation_one_sweep_reaches_every_pair():
    """The effect of the schedule on crafted weights: for every pair of groups (all pairs up to 16
    groups, a seeded sample above), a weight in which only that pair can gain is fixed by one sweep;
    a schedule that skipped the pair would leave the objective at its start."""
    rng = np.random.default_rng(5)
    for G in list(range(2, 17)) + [17, 24, 33, 40]:
        pairs = list(itertools.combinations(range(G), 2))
        if G > 16:
            pick = rng.choice(len(pairs), size=24, replace=False)
            pairs = sorted(set([pairs[i] for i in pick] + [(0, G - 1), (G - 2, G - 1), (0, 1)]))
        for a, b in pairs:
            W = _one_improvable_pair(G, a, b)
            before = oracle.retained(W, oracle.FP32)
            assert before == 2 * (27 + 40 * (G - 2))
            perm = oracle.channel_permutation(W, oracle.FP32, 1)
            assert sorted(perm.tolist()) == list(range(4 * G))
            assert oracle.retained(W, oracle.FP32, perm) == 2 * (36 + 40 * (G - 2)), (G, a, b)


def _pair_gain_left(S, perm):
    """Largest strict gain any pair of groups could still make by re-partitioning its 8 channels
    (numpy, exact for integer scores): S is M x K scores, perm the column order."""
    P = S[:, perm]
    G = P.shape[1] // 4
    worst = 0.0
    for a, b in itertools.combinations(range(G), 2):
        ch = np.concatenate([P[:, 4 * a:4 * a + 4], P[:, 4 * b:4 * b + 4]], axis=1)
        cur = (np.sort(ch[:, :4], axis=1)[:, -2:].sum() + np.sort(ch[:, 4:], axis=1)[:, -2:].sum())
        for A in itertools.combinations(range(8), 4):
            if 0 not in A:
                continue
            B = [c for c in range(8) if c not in A]
            v = np.sort(ch[:, list(A)], axis=1)[:, -2:].sum() + np.sort(ch[:, B], axis=1)[:, -2:].sum()
            worst = max(worst, float(v - cur))
    return worst


@pytest.mark.parametrize("K,score", [(48, oracle.MAGNITUDE), (44, oracle.MAGNITUDE), (40, oracle.WANDA)])
def test_permutation_fixed_point_has_no_improving_pair(K, score):
    """Sweeps until one changes nothing; then no pair of groups (every pair, enumerated in numpy) has a
    split among its 35 that keeps strictly more. Integer weights and power-of-two norms keep every
    sum exact, so the comparison has no rounding."""
    rng = np.random.default_rng(K)
    W = rng.integers(-40, 41, size=(24, K)).astype(np.float32)
    norms = None
    S = np.abs(W.astype(np.float64))
    if score == oracle.WANDA:
        norms = (2.0 ** rng.integers(-2, 3, size=K)).astype(np.float32)
        S = S * norms.astype(np.float64)
    prev = oracle.channel_permutation(W, oracle.FP32, 0, score, norms)
    assert np.array_equal(prev, np.arange(K))
    for sweeps in range(1, 60):
        perm = oracle.channel_permutation(W, oracle.FP32, sweeps, score, norms)
        if np.array_equal(perm, prev):
            break
        prev = perm
    else:
        raise AssertionError("no fixed point within 60 sweeps")
    assert sweeps > 1  # the random start was improvable
    assert _pair_gain_left(S, perm) == 0.0
    assert _pair_gain_left(S, np.arange(K)) > 0.0  # the check does see gains where there are some


@pytest.mark.parametrize("score", [oracle.MAGNITUDE, oracle.WANDA])
def test_permutation_invariants(score):
    W = synth.normal_bf16(31, (64, 256))
    norms = None
    if score == oracle.WANDA:
        norms = np.abs(np.random.default_rng(32).standard_normal(256)).astype(np.float32) + 0.1
    r_prev = oracle.retained(W, oracle.BF16, None, score, norms)
    for sweeps in (1, 2, 3):
        perm = oracle.channel_permutation(W, oracle.BF16, sweeps, score, norms)
        assert sorted(perm.tolist()) == list(range(256))
        r = oracle.retained(W, oracle.BF16, perm, score, norms)
        assert r >= r_prev
        r_prev = r
    assert r_prev > oracle.retained(W, oracle.BF16, None, score, norms)
    # equal magnitudes: nothing strictly gains, the order stays
    same = np.full((8, 64), 0x3F80, np.uint16)
    assert np.array_equal(oracle.channel_permutation(same, oracle.BF16, 2), np.arange(64))


def test_permutation_objective_equals_kept_magnitude():
    # the magnitude objective is the sum of |kept values| of the 2:4 compression of the permuted W
    W = synth.normal_bf16(41, (32, 128))
    perm = oracle.channel_permutation(W, oracle.BF16, 2)
    Wp = np.ascontiguousarray(W[:, perm])
    vals, _, _, _ = compress_rm(Wp, oracle.BF16)
    kept = np.abs(synth.bf16_bits_to_f32(vals).astype(np.float64)).sum()
    assert oracle.retained(W, oracle.BF16, perm) == pytest.approx(kept, rel=1e-12)
    assert oracle.retained(Wp, oracle.BF16) == pytest.approx(kept, rel=1e-12)


# ----------------------------------------------------------------- invariants on random data


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP16, oracle.FP32])
def test_invariants_random(dt):
    rng = np.random.default_rng(100 + dt)
    M, K = 48, 320
    Wf = (rng.standard_normal((M, K)) * 0.02).astype(np.float32)
    if dt == oracle.BF16:
        W, Wd = synth.f32_to_bf16_bits(Wf), synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(Wf))
    elif dt == oracle.FP16:
        W = Wf.astype(np.float16).view(np.uint16)
        Wd = W.view(np.float16).astype(np.float32)
    else:
        W, Wd = Wf, Wf
    vals, meta, vflat, mflat = compress_rm(W, dt)
    assert oracle.meta_bad_nibbles(mflat, M, K, dt) == 0
    pos = top2_by_sort(np.abs(Wd))
    nib = meta_nibbles(meta, K).reshape(-1)
    assert np.array_equal(nib & 3, pos[:, 0]) and np.array_equal(nib >> 2, pos[:, 1])
    dense = oracle.decompress(vflat, mflat, dt, M, K)
    ref = dense_from_positions(W, pos)
    assert np.array_equal(dense, ref)  # decompress(compress(W)) == prune(W), bit-exact
    # min kept magnitude >= max dropped magnitude in every group; exactly two non-zeros per group
    a = np.abs(Wd).reshape(-1, 4)
    keep = np.zeros_like(a, bool)
    np.put_along_axis(keep, pos, True, axis=1)
    assert np.all(np.where(keep, a, np.inf).min(1) >= np.where(keep, -np.inf, a).max(1))
    dd = (dense.view(np.uint16) if dt != oracle.FP32 else dense.view(np.uint32)).reshape(-1, 4)
    assert np.all(np.count_nonzero(dd, axis=1) == 2)
    # idempotent: pruning the pruned matrix changes nothing
    v2, m2 = oracle.prune_compress(dense, dt)
    assert np.array_equal(oracle.decompress(v2, m2, dt, M, K), dense)


def test_fp32_input_bf16_values_round_to_nearest_even():
    rng = np.random.default_rng(5)
    W = rng.standard_normal((16, 64)).astype(np.float32)
    vals32, meta32, _, _ = compress_rm(W, oracle.FP32)
    vals16, meta16, _, _ = compress_rm(W, oracle.FP32, val_dtype=oracle.BF16)
    assert np.array_equal(meta32, meta16)
    assert np.array_equal(vals16, synth.f32_to_bf16_bits(vals32))


def test_fp32_to_bf16_definition_vs_torch():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(20000).astype(np.float32) * np.float32(1e3)
    # exact ties: low 16 bits 0x8000 with both parities of the kept bit
    ties = (rng.integers(0x3F800000, 0x47000000, size=2000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    edge = np.array([0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000, 0x00008000, 0x00018000, 0x3F808000, 0x3F818000,
                     0x80000000, 0x7F800000], dtype=np.uint32)
    allx = np.concatenate([x, ties.view(np.float32), edge.view(np.float32)])
    ours = np.array([oracle.fp32_to_bf16(v) for v in allx], dtype=np.uint16)
    assert np.array_equal(ours, synth.f32_to_bf16_bits(allx))
    assert oracle.fp32_to_bf16(np.float32(1 + 2 ** -8)) == 0x3F80  # tie -> even (1.0)
    assert oracle.fp32_to_bf16(np.float32(1 + 3 * 2 ** -8)) == 0x3F82  # tie -> even (1 + 2^-6)


def test_fp16_decoding_every_pattern_vs_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float64)
    ours = np.array([oracle.fp16_value(int(v)) for v in h])
    finite = ~np.isnan(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.all(np.isnan(ours[~finite]))


# ----------------------------------------------------------------- Wanda scoring


def test_wanda_hand_example():
    # |w| = 1 2 3 4 with input-channel norms 10 1 1 1 -> scores 10 2 3 4 -> keep positions 0 and 3;
    # magnitude alone would keep 2 and 3.
    w = np.array([1, 2, 3, 4, -4, 3, 2, 1] + [0] * 8, dtype=np.float32)
    norms = np.array([10, 1, 1, 1, 0.25, 1, 8, 1] + [1] * 8, dtype=np.float32)  # group 1: 1 3 16 1 -> 1, 2
    _, meta, _, _ = compress_rm(w.reshape(1, 16), oracle.FP32, oracle.WANDA, norms)
    nib = meta_nibbles(meta, 16)[0, :2]
    assert [(n & 3, n >> 2) for n in nib] == [(0, 3), (1, 2)]
    _, meta_m, _, _ = compress_rm(w.reshape(1, 16), oracle.FP32)
    assert [(n & 3, n >> 2) for n in meta_nibbles(meta_m, 16)[0, :2]] == [(2, 3), (0, 1)]


@pytest.mark.parametrize("p", [0, 3, -5])
def test_wanda_with_uniform_power_of_two_norms_equals_magnitude(p):
    rng = np.random.default_rng(11)
    W = synth.f32_to_bf16_bits((rng.standard_normal((32, 128)) * 0.02).astype(np.float32))
    norms = np.full(128, 2.0 ** p, dtype=np.float32)
    a = oracle.prune_compress(W, oracle.BF16, oracle.WANDA, norms)
    b = oracle.prune_compress(W, oracle.BF16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_wanda_vs_sorted_float32_scores():
    rng = np.random.default_rng(12)
    M, K = 40, 256
    W = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 0.02).astype(np.float32))
    norms = (np.exp(rng.standard_normal(K)) * 30).astype(np.float32)
    norms[::7] = norms[1::7][: len(norms[::7])]  # some repeated norms -> more ties
    vals, meta, _, _ = compress_rm(W, oracle.BF16, oracle.WANDA, norms)
    s = np.abs(synth.bf16_bits_to_f32(W)) * norms[None, :]  # float32 * float32 in numpy: one rounding
    assert s.dtype == np.float32
    pos = top2_by_sort(s)
    nib = meta_nibbles(meta, K).reshape(-1)
    assert np.array_equal(nib & 3, pos[:, 0]) and np.array_equal(nib >> 2, pos[:, 1])


def test_wanda_rejects_int8_and_missing_norms():
    with pytest.raises(oracle.OracleError):
        oracle.prune_compress(np.zeros((1, 16), np.int8), oracle.I8, oracle.WANDA, np.ones(16, np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.prune_compress(np.zeros((1, 16), np.float32), oracle.FP32, oracle.WANDA, None)
    with pytest.raises(oracle.OracleError):
        oracle.prune_compress(np.zeros((1, 8), np.float32), oracle.FP32)  # K not a multiple of 16


# ----------------------------------------------------------------- column norms


@pytest.mark.parametrize("p,k", [(0, 0), (3, 1), (-4, 5), (7, 3)])
def test_col_norms_closed_form(p, k):
    N = 4 ** k
    a = np.float32(2.0 ** p)
    X = synth.f32_to_bf16_bits(np.full((3, N), a, dtype=np.float32))
    X[1] = synth.f32_to_bf16_bits(np.full(N, -a, dtype=np.float32))
    out = oracle.col_norms(X)
    assert np.all(out == np.float32(abs(a) * 2.0 ** k))


def test_col_norms_vs_numpy_norm():
    X = synth.heavy_tailed_bf16(9, 64, 2048)
    out = oracle.col_norms(X)
    ref = np.linalg.norm(synth.bf16_bits_to_f32(X).astype(np.float64), axis=1)
    np.testing.assert_allclose(out, ref, rtol=1.2e-7)  # one fp32 rounding of an fp64 result
    # strided view: only the first N columns of each row count
    wide = np.concatenate([X, np.full((64, 8), 0x7F80, np.uint16)], axis=1)  # +inf padding, ignored
    assert np.array_equal(oracle.col_norms(wide[:, :2048]), out)


# ----------------------------------------------------------------- sparse GEMM


def _rand_pruned(seed, M, K, dt=oracle.BF16):
    rng = np.random.default_rng(seed)
    W = synth.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    vals, meta = oracle.prune_compress(W, dt)
    return W, vals, meta


@pytest.mark.parametrize("M,K,N", [(16, 16, 1), (37, 64, 29), (64, 48, 64), (5, 128, 3), (40, 208, 7)])
def test_gemm_bf16_vs_numpy_matmul(M, K, N):
    W, vals, meta = _rand_pruned(M * 1000 + K + N, M, K)
    X = synth.normal_bf16(N + 17, (K, N))
    pos = top2_by_sort(np.abs(synth.bf16_bits_to_f32(W)))
    Wp = synth.bf16_bits_to_f32(dense_from_positions(W, pos)).astype(np.float64)
    ref = Wp @ synth.bf16_bits_to_f32(X).astype(np.float64)
    Y = oracle.gemm_bf16(vals, meta, X, M)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)
    rows = np.array([M - 1, 0, M // 2])
    assert np.array_equal(oracle.gemm_bf16(vals, meta, X, M, rows=rows), Y[rows])


def test_gemm_bf16_identity_equals_decompress():
    M, K = 24, 64
    W, vals, meta = _rand_pruned(4, M, K)
    eye = synth.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    Y = oracle.gemm_bf16(vals, meta, eye, M)
    dense = synth.bf16_bits_to_f32(oracle.decompress(vals, meta, oracle.BF16, M, K)).astype(np.float64)
    assert np.array_equal(Y, dense)


def test_gemm_bf16_one_hot_columns_select_columns():
    M, K = 16, 32
    W, vals, meta = _rand_pruned(6, M, K)
    cols = [3, 0, 31, 17]
    X = np.zeros((K, len(cols)), np.float32)
    for j, c in enumerate(cols):
        X[c, j] = 1.0
    Y = oracle.gemm_bf16(vals, meta, synth.f32_to_bf16_bits(X), M)
    dense = synth.bf16_bits_to_f32(oracle.decompress(vals, meta, oracle.BF16, M, K)).astype(np.float64)
    assert np.array_equal(Y, dense[:, cols])


def test_gemm_i8_vs_numpy_integer_matmul_and_dequant():
    rng = np.random.default_rng(8)
    M, K, N = 33, 96, 40
    W = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(K, N), dtype=np.int8)
    vals, meta = oracle.prune_compress(W, oracle.I8)
    pos = top2_by_sort(np.abs(W.astype(np.int32)))
    Wp = dense_from_positions(W, pos).astype(np.int64)
    ref = Wp @ X.astype(np.int64)
    scale = (rng.random(M) * 1e-3).astype(np.float32)
    acc, Y = oracle.gemm_i8(vals, meta, X, M, scale)
    assert np.array_equal(acc, ref)
    assert np.array_equal(Y, ref.astype(np.int32).astype(np.float32) * scale[:, None])
    acc2, Y2 = oracle.gemm_i8(vals, meta, X, M)
    assert Y2 is None and np.array_equal(acc2, ref)


@pytest.mark.parametrize("M,K,N", [(16, 16, 1), (37, 64, 29), (5, 128, 3)])
def test_gemm_bf16_token_major_vs_numpy_matmul(M, K, N):
    # a Linear layer's orientation: Y (N x M) = X (N x K) @ Wp^T, by numpy in that orientation
    W, vals, meta = _rand_pruned(M * 7 + K + N, M, K)
    X = synth.normal_bf16(N + 31, (N, K))
    pos = top2_by_sort(np.abs(synth.bf16_bits_to_f32(W)))
    Wp = synth.bf16_bits_to_f32(dense_from_positions(W, pos)).astype(np.float64)
    ref = synth.bf16_bits_to_f32(X).astype(np.float64) @ Wp.T
    Y = oracle.gemm_bf16(vals, meta, X, M, layout="token")
    assert Y.shape == (N, M)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)
    rows = np.array([M - 1, 0])
    assert np.array_equal(oracle.gemm_bf16(vals, meta, X, M, rows=rows, layout="token"), Y[:, rows])


def test_gemm_i8_token_major_vs_numpy_integer_matmul():
    rng = np.random.default_rng(81)
    M, K, N = 20, 64, 9
    W = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    X = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
    vals, meta = oracle.prune_compress(W, oracle.I8)
    Wp = dense_from_positions(W, top2_by_sort(np.abs(W.astype(np.int32)))).astype(np.int64)
    ref = X.astype(np.int64) @ Wp.T
    scale = (rng.random(M) * 1e-3).astype(np.float32)
    acc, Y = oracle.gemm_i8(vals, meta, X, M, scale, layout="token")
    assert np.array_equal(acc, ref)
    assert np.array_equal(Y, ref.astype(np.int32).astype(np.float32) * scale[None, :])


def test_gelu_reference_vs_torch_and_identities():
    # the fused epilogue's GELU reference against torch's exact (erf) GELU in float64
    x = np.concatenate([np.linspace(-12, 12, 2001), [0.0, 1e-30, -1e-30, 1e-8, -40.0, 40.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="none").numpy()
    # (1 + erf) cancels for large negative x in both: compare with an absolute floor there
    np.testing.assert_allclose(oracle.gelu64(x), ref, rtol=1e-14, atol=1e-15)
    # GELU(x) - GELU(-x) = x, GELU(0) = 0, GELU(x) -> x for large x
    np.testing.assert_allclose(oracle.gelu64(x) - oracle.gelu64(-x), x, rtol=1e-14, atol=1e-15)
    assert oracle.gelu64(0.0) == 0.0 and oracle.gelu64(40.0) == 40.0


def test_requant_rule_examples():
    # clamp(rne(y * fl32(1/s)), -127, 127): halfway cases to even, clamping at +-127 (never -128)
    y = np.array([2.5, 3.5, -2.5, -3.5, 127.6, 126.5, -300.0, 0.49999997, -0.5, 0.0], np.float32)
    assert oracle.requant_i8(y, 1.0).tolist() == [2, 4, -2, -4, 127, 126, -127, 0, 0, 0]
    # the reciprocal is rounded to fp32 first: fl32(1/0.1f) = 10 exactly, fl32(0.25 * 10) = 2.5 -> 2
    assert np.float32(1) / np.float32(0.1) == np.float32(10.0)
    assert oracle.requant_i8(np.float32(0.25), 0.1).item() == 2
    # fl32(1/3) = 0.33333334: 7.5 and 4.5 times it round to exactly 2.5 and 1.5 in fp32, then to even
    assert oracle.requant_i8(np.array([7.5, 4.5], np.float32), 3.0).tolist() == [2, 2]
    # in float64 the products stay above the halfway points: 2.5000000 + 5e-8 -> 3, 1.5 + 3e-8 -> 2
    assert oracle.requant_i8(np.array([7.5, 4.5], np.float64), 3.0).tolist() == [3, 2]


def test_gemm_i8_fused_closed_forms():
    rng = np.random.default_rng(90)
    M, K, N = 24, 64, 11
    W = rng.integers(-3, 4, size=(M, K), dtype=np.int8)
    X = rng.integers(-3, 4, size=(K, N), dtype=np.int8)
    vals, meta = oracle.prune_compress(W, oracle.I8)
    acc, _ = oracle.gemm_i8(vals, meta, X, M)
    one = np.ones(M, np.float32)
    bias = rng.integers(-20, 21, size=M).astype(np.float32)
    # scale 1 and integer bias: every step is exact, y = acc + bias
    r = oracle.gemm_i8_fused(vals, meta, X, M, one, bias, out_scale=1.0)
    assert np.array_equal(r["y32"], (acc + bias[:, None]).astype(np.float32))
    assert np.array_equal(r["q"], np.clip(acc + bias[:, None], -127, 127).astype(np.int8))
    # GELU of exact integers against torch
    g = oracle.gemm_i8_fused(vals, meta, X, M, one, bias, gelu=True)["y"]
    ref = torch.nn.functional.gelu(torch.from_numpy((acc + bias[:, None]).astype(np.float64))).numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-300)
    # no bias, no GELU: the plain dequantized GEMM
    s = (rng.random(M) * 1e-2).astype(np.float32)
    assert np.array_equal(oracle.gemm_i8_fused(vals, meta, X, M, s)["y"], oracle.gemm_i8(vals, meta, X, M, s)[1])
    # token-major layout: the transpose
    rt = oracle.gemm_i8_fused(vals, meta, np.ascontiguousarray(X.T), M, one, bias, out_scale=1.0, layout="token")
    assert np.array_equal(rt["q"], r["q"].T)


def test_gemm_i8_overflow_is_reported():
    K = 270000 - 270000 % 16
    W = np.full((1, K), -128, np.int8)
    X = np.full((K, 1), -128, np.int8)
    vals, meta = oracle.prune_compress(W, oracle.I8)
    with pytest.raises(oracle.OracleError):
        oracle.gemm_i8(vals, meta, X, 1)


def test_noncanonical_metadata_is_rejected():
    vals, meta = oracle.prune_compress(np.ones((3, 16), np.uint16), oracle.BF16)
    for bad in (0x00, 0x5, 0x1, 0x6, 0xF):  # i0 == i1 or i0 > i1
        m = meta.copy()
        off = oracle.meta_offset(2, 1, 16, oracle.BF16)  # row 2, groups 2 and 3
        m[off] = bad | (0x4 << 4)
        assert oracle.meta_bad_nibbles(m, 3, 16, oracle.BF16) == 1
        with pytest.raises(oracle.OracleError):
            oracle.decompress(vals, m, oracle.BF16, 3, 16)


# ----------------------------------------------------------------- int8 preparation (caller side)


def test_int8_row_scale_covers_9999_and_pruned_equals_unpruned():
    W = synth.normal_f32(21, (64, 768), 0.02)
    vals, meta = oracle.prune_compress(W, oracle.FP32)
    Wp = oracle.decompress(vals, meta, oracle.FP32, *W.shape)
    q, s = synth.quantize_rows(Wp)
    q0, s0 = synth.quantize_rows(W)
    assert np.array_equal(s, s0)  # the 0.9999 quantile of 768 values sits between the top two
    assert q.min() >= -127 and q.max() <= 127
    # s is the 0.9999 quantile over 127, rounded once to fp32; only the values above that quantile
    # (at most K - 1 - floor(0.9999 (K - 1)) of them per row, 1 for K = 768) get clipped
    K = W.shape[1]
    qtl = np.quantile(np.abs(Wp).astype(np.float64), 0.9999, axis=1)
    np.testing.assert_allclose(s.astype(np.float64), qtl / 127, rtol=2.0 ** -24)
    above = np.sum(np.abs(Wp) > qtl[:, None], axis=1)
    assert np.all(above <= K - 1 - np.floor(0.9999 * (K - 1)))
    # round half to even on exact ties
    assert synth.quantize_sym(np.array([0.5, 1.5, 2.5, -0.5]), np.float32(1.0)).tolist() == [0, 2, 2, 0]
    # quantizing the pruned matrix and re-pruning by |q| keeps the dense int8 matrix unchanged
    v8, m8 = oracle.prune_compress(q, oracle.I8)
    assert np.array_equal(oracle.decompress(v8, m8, oracle.I8, *q.shape), q)


# ----------------------------------------------------------------- compressed layout


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP32, oracle.I8])
@pytest.mark.parametrize("M,K", [(1, 16), (16, 64), (37, 208), (48, 384)])
def test_layout_offsets_match_the_stated_layout(dt, M, K):
    from tests.layout_ref import _perm, padded_shape
    e = ESIZE[dt]
    Mp, Kp = padded_shape(M, K, e)
    vb, mb = oracle.compressed_bytes(M, K, dt)
    assert (vb, mb) == (Mp * Kp // 2 * e, Mp * Kp // 8)
    pv = _perm(Mp, Kp // 2 * e, 64)
    pm = _perm(Mp, Kp // 8, 16 // e)
    assert sorted(pv.ravel().tolist()) == list(range(vb))  # a permutation of the buffer
    for i in sorted({0, M - 1, Mp - 1, min(17, Mp - 1)}):
        for b in sorted({0, 15, 16, 63, 64, Kp // 2 * e - 1} & set(range(Kp // 2 * e))):
            assert oracle.values_offset(i, b, K, dt) == pv[i, b]
        for b in sorted({0, 1, 3, Kp // 8 - 1} & set(range(Kp // 8))):
            assert oracle.meta_offset(i, b, K, dt) == pm[i, b]


def test_layout_one_tile_is_the_smfmac_operand_order():
    # a 16 x 64 bf16 weight is one tile: lane l = 16 q + r of v_smfmac_f32_16x16x64_bf16 holds the
    # 8 kept values of row r, dense columns [16 q, 16 q + 16), at bytes [16 l, 16 l + 16)
    W = synth.normal_bf16(3, (16, 64))
    vflat, mflat = oracle.prune_compress(W, oracle.BF16)
    vr, mr = to_row_major(vflat, mflat, 16, 64, 2)
    for lane in range(64):
        q, r = lane // 16, lane % 16
        assert np.array_equal(vflat[8 * lane: 8 * lane + 8], vr[r, 8 * q: 8 * q + 8])
        assert mflat[2 * lane: 2 * lane + 2].tolist() == mr[r, 2 * q: 2 * q + 2].tolist()
