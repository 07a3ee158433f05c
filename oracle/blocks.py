"""Spatio-temporal block order of a step's tokens (oracle, test infrastructure).

Ultra Flash notes, key design 3: the 3-D token grid (frames, rows, columns) is
cut into non-overlapping (2, 8, 8) blocks of 128 tokens, the unit of the
block-sparse mask.  The notes give no rule for grids that these blocks do not
tile (60x104 and 90x156 token frames, 3-frame chunks).  Read here, for the F
frames of one step with an H x W grid:
  1. frame pairs (0, 1), (2, 3), ...: every full (2, 8, 8) block, blocks in
     row-major order of their (block row, block column), tokens inside a block
     frame first, then row, then column;
  2. if F is odd, the last frame: every full 8 x 8 patch, patches in the same
     order, tokens row then column (two consecutive patches fill one tile);
  3. then every token outside a full block or patch (rows from 8*floor(H/8)
     on, or columns from 8*floor(W/8) on), in raster order: frame, row, column.
The order is built here by listing the tokens region by region; position i
of the block order holds raster token order[i] (= frame*H*W + row*W + column).
"""
from __future__ import annotations

import numpy as np


def block_order(frames: int, grid_h: int, grid_w: int) -> np.ndarray:
    """Raster token index at each position of the step's block order (a permutation)."""
    if frames < 1 or grid_h < 1 or grid_w < 1:
        raise ValueError("bad step shape")
    hb, wb = grid_h // 8, grid_w // 8
    out = []

    def raster(f, y, x):
        return (f * grid_h + y) * grid_w + x

    for p in range(frames // 2):
        for by in range(hb):
            for bx in range(wb):
                for t in (2 * p, 2 * p + 1):
                    for y in range(8 * by, 8 * by + 8):
                        for x in range(8 * bx, 8 * bx + 8):
                            out.append(raster(t, y, x))
    if frames % 2:
        f = frames - 1
        for by in range(hb):
            for bx in range(wb):
                for y in range(8 * by, 8 * by + 8):
                    for x in range(8 * bx, 8 * bx + 8):
                        out.append(raster(f, y, x))
    for f in range(frames):
        for y in range(grid_h):
            for x in range(grid_w):
                if y >= 8 * hb or x >= 8 * wb:
                    out.append(raster(f, y, x))
    return np.asarray(out, dtype=np.int64)


def to_block_order(x: np.ndarray, frames: int, grid_h: int, grid_w: int) -> np.ndarray:
    """Rows of x (a step's tokens in raster order) rearranged into block order."""
    return x[block_order(frames, grid_h, grid_w)]


def from_block_order(x: np.ndarray, frames: int, grid_h: int, grid_w: int) -> np.ndarray:
    """Inverse of to_block_order."""
    out = np.empty_like(x)
    out[block_order(frames, grid_h, grid_w)] = x
    return out
