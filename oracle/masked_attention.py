"""Masked softmax attention with GQA head sharing.

For every batch item b and query head h, with KV head g = h // (Hq / Hkv) (consecutive
query heads share one KV head; hidream-o1-p100a model card, "GQA 32/8"):
    Z = Q_bh K_bg^T * scale,  Z[~M_b] = -inf,  P = softmax_rows(Z),  O_bh = P V_bg.
scale defaults to 1/sqrt(d). Computed in float64 (or the dtype asked for), in row chunks
to bound memory; chunking changes nothing but the order of independent rows.
"""
from __future__ import annotations

import numpy as np


def _softmax_rows(z: np.ndarray) -> np.ndarray:
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, masks, scale=None, dtype=np.float64, heads=None, row_chunk=1024):
    """q [B][S][Hq][d], k/v [B][S][Hkv][d], masks [B][S][S] bool -> out [B][S][Hq][d].

    heads: optional iterable of query heads to compute (others are left as NaN)."""
    q = np.asarray(q)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    out = np.full((B, S, Hq, d), np.nan, dtype=dtype)
    heads = range(Hq) if heads is None else heads
    for b in range(B):
        M = masks[b]
        for h in heads:
            g = h // group
            K = np.asarray(k[b, :, g, :], dtype=dtype)
            V = np.asarray(v[b, :, g, :], dtype=dtype)
            for r0 in range(0, S, row_chunk):
                r1 = min(S, r0 + row_chunk)
                Q = np.asarray(q[b, r0:r1, h, :], dtype=dtype)
                Z = (Q @ K.T) * dtype(scale)
                Z = np.where(M[r0:r1], Z, -np.inf)
                out[b, r0:r1, h, :] = _softmax_rows(Z) @ V
    return out


def attention_rows(q, k, v, mask_rows, rows, heads, scale=None, dtype=np.float64):
    """Selected outputs: rows [n] (query token indices) x heads [m] of one batch item.

    q [S][Hq][d], k/v [S][Hkv][d] of that item, mask_rows [n][S] bool -> [n][m][d]."""
    S, Hq, d = q.shape
    group = Hq // k.shape[1]
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    rows = np.asarray(rows)
    out = np.empty((len(rows), len(heads), d), dtype=dtype)
    for hi, h in enumerate(heads):
        g = h // group
        K = np.asarray(k[:, g, :], dtype=dtype)
        V = np.asarray(v[:, g, :], dtype=dtype)
        Q = np.asarray(q[rows, h, :], dtype=dtype)
        Z = (Q @ K.T) * dtype(scale)
        Z = np.where(mask_rows, Z, -np.inf)
        out[:, hi, :] = _softmax_rows(Z) @ V
    return out
