"""Tiled storage layout of expert matrices, written out as index arithmetic. TEST INFRASTRUCTURE
ONLY (the same import rules as the rest of this package).

The verify pass streams every woken expert's bytes once per block ([SH2], section "The
verification cog"), so the library keeps expert matrices in the order its matrix-core tiles
consume them. This module states that order from its definition, with no reference to the GPU
code: a matrix W[R][C] (C the reduction dimension) is cut into tiles of 16 rows x 32 columns;
inside a tile, slice l (0..63) holds row l % 16, columns 8 (l // 16) .. 8 (l // 16) + 7; tiles
run column-step-major within a 16-row band, bands in row order. For mxfp4 the unit is the 32-value
block (16 code bytes, one scale byte): slice l of window w (4 blocks) in band rt holds block
4 w + l // 16 of row 16 rt + l % 16.
"""
from __future__ import annotations

import numpy as np


def tile_bf16(w: np.ndarray) -> np.ndarray:
    """[n][R][C] (or [R][C]) 16-bit words -> the same shape, holding the tiled order row-major."""
    a = w if w.ndim == 3 else w[None]
    n, R, C = a.shape
    assert R % 16 == 0 and C % 128 == 0
    t = a.reshape(n, R // 16, 16, C // 32, 4, 8)        # band, row-in-band, step, quarter, elem
    t = t.transpose(0, 1, 3, 4, 2, 5)                   # band, step, quarter, row-in-band, elem
    return np.ascontiguousarray(t).reshape(a.shape if w.ndim == 3 else w.shape)


def tile_mxfp4(codes: np.ndarray, scales: np.ndarray):
    """codes [n][R][C/2] bytes and scales [n][R][C/32] -> both in the tiled order, same shapes."""
    c = codes if codes.ndim == 3 else codes[None]
    s = scales if scales.ndim == 3 else scales[None]
    n, R, half = c.shape
    C = half * 2
    assert R % 16 == 0 and C % 128 == 0 and s.shape == (n, R, C // 32)
    tc = c.reshape(n, R // 16, 16, C // 128, 4, 16).transpose(0, 1, 3, 4, 2, 5)   # band, window, q, row, byte
    ts = s.reshape(n, R // 16, 16, C // 128, 4).transpose(0, 1, 3, 4, 2)           # band, window, q, row
    return (np.ascontiguousarray(tc).reshape(codes.shape), np.ascontiguousarray(ts).reshape(scales.shape))


def tiled_position_bf16(R: int, C: int, row: int, col: int) -> int:
    """Element index, in the flat tiled array of one R x C matrix, of W[row][col]."""
    band, r = divmod(row, 16)
    step, within = divmod(col, 32)
    q, i = divmod(within, 8)
    return ((band * (C // 32) + step) * 64 + (r + 16 * q)) * 8 + i
