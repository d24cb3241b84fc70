"""Host checks, in numpy fp32 arithmetic, of arithmetic identities the HIP kernels rely on.

Requantization to int8 (the fused epilogue's int8 output): the kernels compute clamp(rne(t), -127, 127) for
t = fl32(y * inv_scale) as the low byte of the float bits of med3(fl32(t + 1.5 * 2^23), B - 127, B + 127).
Here that form is evaluated with numpy's IEEE fp32 add (round to nearest even, as on the GPU) and compared with
the plain definition over ties, the clamp edges, the whole range where the add is exact, and beyond it.
"""
import numpy as np

B = np.float32(12582912.0)  # 1.5 * 2^23


def _kernel_form(t):
    u = (t.astype(np.float32) + B).astype(np.float32)
    c = np.minimum(np.maximum(u, B - np.float32(127)), B + np.float32(127))
    return (c.view(np.uint32) & 0xFF).astype(np.uint8)


def _definition(t):
    q = np.clip(np.rint(t.astype(np.float64)), -127, 127).astype(np.int64)
    return (q & 0xFF).astype(np.uint8)


def test_requant_ties_and_clamp_edges():
    k = np.arange(-140, 141, dtype=np.float32)
    t = np.concatenate([k, k + np.float32(0.5), k - np.float32(0.5), k + np.float32(0.49999997),
                        k - np.float32(0.49999997), np.float32([0.0, -0.0, 126.5, 127.5, -126.5, -127.5,
                                                                 np.inf, -np.inf, 3e38, -3e38, 1e-45, -1e-45])])
    assert np.array_equal(_kernel_form(t), _definition(t))


def test_requant_dense_and_wide_ranges():
    rng = np.random.default_rng(0)
    # every float spacing of interest: small values, the clamp region, up to and past 2^22 where the add
    # stops being exact, and huge magnitudes
    parts = [rng.uniform(-200, 200, 2_000_000), rng.uniform(-2.0 ** 23, 2.0 ** 23, 1_000_000),
             rng.standard_normal(1_000_000) * 1e30, np.float32(2.0 ** 22) + np.arange(-64, 64),
             -np.float32(2.0 ** 22) + np.arange(-64, 64)]
    t = np.concatenate(parts).astype(np.float32)
    assert np.array_equal(_kernel_form(t), _definition(t))


# int8 magnitude selection (the int8 prune): two groups of four int8 weights, one 32-bit word each, go through
# per-byte |q|, keys (|q| << 2) | (3 - e) packed one group per 16-bit half, and packed 16-bit max / min. The
# emulation below follows those steps on uint32 arrays; the reference picks the two largest |q| of each group
# with the lower position first on ties, by sorting.

def _abs_i8x4(w):
    hb = w & np.uint32(0x80808080)
    sgn = hb >> np.uint32(7)
    return ((w ^ ((hb << np.uint32(1)) - sgn)) + sgn).astype(np.uint32)


def _max16(a, b):
    lo = np.maximum(a & np.uint32(0xFFFF), b & np.uint32(0xFFFF))
    hi = np.maximum(a >> np.uint32(16), b >> np.uint32(16))
    return (lo | (hi << np.uint32(16))).astype(np.uint32)


def _min16(a, b):
    lo = np.minimum(a & np.uint32(0xFFFF), b & np.uint32(0xFFFF))
    hi = np.minimum(a >> np.uint32(16), b >> np.uint32(16))
    return (lo | (hi << np.uint32(16))).astype(np.uint32)


def _top2_pair(w0, w1):
    a0, a1 = _abs_i8x4(w0), _abs_i8x4(w1)
    k = []
    for e in range(4):
        b = ((a0 >> np.uint32(8 * e)) & np.uint32(0xFF)) | (((a1 >> np.uint32(8 * e)) & np.uint32(0xFF)) << np.uint32(16))
        k.append(((b << np.uint32(2)) | np.uint32((3 - e) * 0x10001)).astype(np.uint32))
    m01 = _max16(k[0], k[1])
    m3 = _max16(m01, k[2])
    med = _max16(_min16(k[0], k[1]), _min16(m01, k[2]))
    first, second = _max16(m3, k[3]), _max16(med, _min16(m3, k[3]))
    pf, ps = first & np.uint32(0x30003), second & np.uint32(0x30003)
    return _max16(pf, ps) ^ np.uint32(0x30003), _min16(pf, ps) ^ np.uint32(0x30003)


def _top2_reference(w):
    q = np.ascontiguousarray(w).view(np.int8).reshape(-1, 4).astype(np.int64)
    # sort by |q| descending, then position ascending; keep the first two positions, in order
    pos = np.arange(4)[None, :].repeat(len(q), 0)
    order = np.lexsort((pos, -np.abs(q)), axis=1)[:, :2]
    return np.sort(order, axis=1)


def test_int8_pair_selection_matches_sorting():
    rng = np.random.default_rng(5)
    n = 1_000_000
    # random bytes, narrow ranges (many ties), -128, and equal magnitudes of opposite sign
    parts = [rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32),
             rng.integers(-2, 3, (n, 4)).astype(np.int8).view(np.uint32).ravel(),
             rng.choice(np.array([-128, 127, -127, 0, 1, -1], np.int8), (n, 4)).view(np.uint32).ravel()]
    w = np.concatenate(parts)
    w0, w1 = w[0::2], w[1::2]
    lo, hi = _top2_pair(w0, w1)
    ref0, ref1 = _top2_reference(w0), _top2_reference(w1)
    assert np.array_equal(lo & np.uint32(0xFFFF), ref0[:, 0]) and np.array_equal(hi & np.uint32(0xFFFF), ref0[:, 1])
    assert np.array_equal(lo >> np.uint32(16), ref1[:, 0]) and np.array_equal(hi >> np.uint32(16), ref1[:, 1])
