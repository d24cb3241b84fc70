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
