"""Rotary position embedding: 1D, generalized 2D, and 3-axis interleaved mRoPE.

1D RoPE (HunyuanImage 3.0 digest, "Generalized 2D Rotary Position Embedding"): a position
n rotates the query/key by angles n * theta_i, one frequency per pair, with features laid
out as all cosines then all sines; scores then depend only on the relative position.
Readings: d/2 frequencies theta_i = base^(-2i/d), i = 0 .. d/2-1 (the page's list
{theta_0 .. theta_{d/2}} has one item too many); "all cosines then all sines" means the
pair for frequency i is (x[i], x[i + d/2]) (rotate-half layout).

Generalized 2D RoPE (same section): position (x, y) uses cos(x theta_0), cos(y theta_1),
... i.e. the frequencies alternate between the two axes. The prose of the same page says
the first half encodes x and the second half y; the printed formula is followed here:
pair i even -> axis 0 (x, horizontal), i odd -> axis 1 (y, vertical). Text sits on the
diagonal (n, n), so with no image tokens this reduces exactly to 1D RoPE.

mRoPE (hidream-o1-p100a model card, architecture paragraph): "3-axis interleaved mRoPE
[24,20,20] at theta 5e6". Reading: pairs are dealt to the axes (T, H, W) in turn, an axis
dropping out of the rotation once it holds its section count; for [24,20,20] that is
pair i -> i mod 3 for i < 60 and T for pairs 60..63.

Positions are inputs ([B][S][n_axes] integers); pair i uses the position on its axis.
"""
from __future__ import annotations

import numpy as np


def inv_freq(base: float, head_dim: int) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / head_dim)


def axis_of_pair(kind: str, head_dim: int, sections=(0, 0, 0)) -> np.ndarray:
    half = head_dim // 2
    if kind in ("none", "1d"):
        return np.zeros(half, dtype=np.int64)
    if kind == "2d":
        return np.arange(half, dtype=np.int64) % 2
    if kind == "mrope":
        if sum(sections) != half:
            raise ValueError("mRoPE sections must sum to head_dim / 2")
        left = list(sections)
        out = []
        axis = 0
        while len(out) < half:
            if left[axis] > 0:
                out.append(axis)
                left[axis] -= 1
            axis = (axis + 1) % 3
        return np.asarray(out, dtype=np.int64)
    raise ValueError(f"unknown rotary kind {kind}")


def rope_angles(positions: np.ndarray, axes: np.ndarray, freqs: np.ndarray) -> np.ndarray:
    """fp64 angles [B][S][d/2]: position on pair i's axis times frequency i."""
    pos = np.asarray(positions, dtype=np.float64)
    return pos[..., axes] * freqs


def apply_rope(x: np.ndarray, angles: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Rotate each (x[i], x[i + d/2]) pair of every head by its angle.

    x: [B][S][H][d]; angles: [B][S][d/2] (shared by all heads of a token)."""
    x = np.asarray(x, dtype=dtype)
    half = x.shape[-1] // 2
    c = np.cos(angles).astype(dtype)[:, :, None, :]
    s = np.sin(angles).astype(dtype)[:, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
