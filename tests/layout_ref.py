"""Independent numpy statement of the compressed layout (tests only).

Compressed row i of an M x K weight has K/2 kept values and K/8 metadata bytes. Rows are padded to
a multiple of 16 and columns to KT = 128 / e dense columns (e = value size in bytes). The values and
metadata are stored as 16-row tiles (64 bytes of values, KT/8 bytes of metadata per row), row blocks
outer and K tiles inner; inside a tile each row is cut into 4 equal quarters stored quarter-major
(quarter 0 of rows 0..15, then quarter 1, ...). Padding holds value 0 and metadata nibble 0x4.
"""
import numpy as np


def padded_shape(M, K, esize):
    kt = 128 // esize
    return (M + 15) // 16 * 16, (K + kt - 1) // kt * kt


def _perm(Mp, row_bytes, tile_bytes):
    """offset[i, b] of byte b of padded row i for tiles of `tile_bytes` per row."""
    i = np.arange(Mp)[:, None]
    b = np.arange(row_bytes)[None, :]
    q = tile_bytes // 4
    tiles_per_row = row_bytes // tile_bytes
    rb, r = i // 16, i % 16
    t, c, o = b // tile_bytes, (b % tile_bytes) // q, b % q
    return ((rb * tiles_per_row + t) * 4 + c) * (16 * q) + r * q + o


def to_row_major(values_flat, meta_flat, M, K, esize):
    """(values M x K/2 elements, meta M x K/8 bytes) row-major views of the compressed buffers."""
    Mp, Kp = padded_shape(M, K, esize)
    vb = np.ascontiguousarray(values_flat).view(np.uint8)
    mb = np.ascontiguousarray(meta_flat).view(np.uint8)
    assert vb.size == Mp * Kp // 2 * esize and mb.size == Mp * Kp // 8
    v_rm = vb[_perm(Mp, Kp // 2 * esize, 64)]
    m_rm = mb[_perm(Mp, Kp // 8, 16 // esize)]
    vals = v_rm.reshape(Mp, -1).copy().view(np.asarray(values_flat).dtype)[:M, : K // 2]
    return vals, m_rm[:M, : K // 8]


def padding_ok(values_flat, meta_flat, M, K, esize):
    """True when every padded slot holds value 0 and metadata nibble 0x4."""
    Mp, Kp = padded_shape(M, K, esize)
    vb = np.ascontiguousarray(values_flat).view(np.uint8)
    mb = np.ascontiguousarray(meta_flat).view(np.uint8)
    v_rm = vb[_perm(Mp, Kp // 2 * esize, 64)]
    m_rm = mb[_perm(Mp, Kp // 8, 16 // esize)]
    vmask = np.ones_like(v_rm, bool)
    vmask[:M, : K // 2 * esize] = False
    mmask = np.ones_like(m_rm, bool)
    mmask[:M, : K // 8] = False
    return bool(np.all(v_rm[vmask] == 0) and np.all(m_rm[mmask] == 0x44))
