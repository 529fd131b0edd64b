"""Tile labels by brute force over the explicit mask.

The key/query plane is cut into tiles of block_q query rows by block_k key columns,
starting at index 0; the last row and column of tiles may be ragged. Over the valid part
of a tile (rows and columns < S):
  SKIP (0)     no allowed pair,
  FULL (1)     every pair allowed,
  PARTIAL (2)  anything else.
This is the definition itself, evaluated on every element; it does not use any
per-row shortcut.
"""
from __future__ import annotations

import numpy as np


def tile_labels(mask: np.ndarray, block_q: int, block_k: int) -> np.ndarray:
    S = mask.shape[0]
    nq = -(-S // block_q)
    nk = -(-S // block_k)
    out = np.empty((nq, nk), dtype=np.uint8)
    for qb in range(nq):
        for kb in range(nk):
            t = mask[qb * block_q:(qb + 1) * block_q, kb * block_k:(kb + 1) * block_k]
            if not t.any():
                out[qb, kb] = 0
            elif t.all():
                out[qb, kb] = 1
            else:
                out[qb, kb] = 2
    return out
