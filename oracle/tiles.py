"""Tile labels by brute force over the explicit mask.

The key/query plane is cut into tiles of block_q query rows by block_k key columns. Key
tiles start at index 0 (the last one may be ragged). Query blocks start at index 0 too,
or, with q_end_aligned, are cut back from the end of the sequence: block qb then covers
rows [S - (nq - qb) * block_q, S - (nq - qb - 1) * block_q), clipped at 0, so the first
block is the ragged one. Over the valid part of a tile (rows and columns in [0, S)):
  SKIP (0)     no allowed pair,
  FULL (1)     every pair allowed,
  PARTIAL (2)  anything else.
This is the definition itself, evaluated on every element; it does not use any
per-row shortcut.
"""
from __future__ import annotations

import numpy as np


def tile_labels(mask: np.ndarray, block_q: int, block_k: int,
                q_end_aligned: bool = False) -> np.ndarray:
    S = mask.shape[0]
    nq = -(-S // block_q)
    nk = -(-S // block_k)
    q0 = S - nq * block_q if q_end_aligned else 0
    out = np.empty((nq, nk), dtype=np.uint8)
    for qb in range(nq):
        r0, r1 = max(q0 + qb * block_q, 0), q0 + (qb + 1) * block_q
        for kb in range(nk):
            t = mask[r0:r1, kb * block_k:(kb + 1) * block_k]
            if not t.any():
                out[qb, kb] = 0
            elif t.all():
                out[qb, kb] = 1
            else:
                out[qb, kb] = 2
    return out
