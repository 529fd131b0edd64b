"""Seeded input generation.

Draw recipe: numpy Generator(PCG64(seed)), drawing in the fixed order q, k, v, w_q, w_k.
q, k, v ~ N(0, 1) drawn in fp32; for bf16 workloads each draw is rounded to the nearest
bf16 (ties to even) and the upcast of that bf16 is what both sides consume. q/k norm
weights are 1 + 0.02 * N(0, 1) in fp32 (only when the workload enables q/k RMSNorm).

Positions (an input of the path, not computed by it): a text token at sequence index n
gets n on every axis. A patch (r, c) of an image segment that starts at index s0 gets
  2 axes: (x, y) = (s0 + c, s0 + r)       x horizontal (column), y vertical (row)
  3 axes: (T, H, W) = (s0, s0 + r, s0 + c)
so image coordinates sit between the positions of the text around the segment, as the
HunyuanImage 3.0 digest describes for generalized 2D RoPE ("Generalized 2D Rotary
Position Embedding", backward compatibility paragraph). With one axis every token gets
its sequence index.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import Workload


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the 16-bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += b
    t >>= np.uint32(16)
    return t.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
    t <<= np.uint32(16)
    return t.view(np.float32)


def segment_table(w: Workload) -> np.ndarray:
    """int32 [batch][n_segments][3] rows of (start, length, kind), same layout per batch item."""
    rows = []
    start = 0
    for s in w.segments:
        rows.append((start, s.length, s.kind))
        start += s.length
    t = np.asarray(rows, dtype=np.int32).reshape(1, len(rows), 3)
    return np.ascontiguousarray(np.repeat(t, w.batch, axis=0))


def positions_for(w: Workload) -> np.ndarray:
    """int32 [batch][seq_len][n_axes] position ids (recipe in the module docstring)."""
    S, A = w.seq_len, w.n_axes
    pos = np.empty((S, A), dtype=np.int32)
    s0 = 0
    for seg in w.segments:
        idx = np.arange(s0, s0 + seg.length, dtype=np.int64)
        if seg.grid is None or A == 1:
            pos[s0:s0 + seg.length, :] = idx[:, None]
        else:
            rows, cols = seg.grid
            r = (idx - s0) // cols
            c = (idx - s0) % cols
            if A == 2:
                pos[s0:s0 + seg.length, 0] = s0 + c
                pos[s0:s0 + seg.length, 1] = s0 + r
            else:
                pos[s0:s0 + seg.length, 0] = s0
                pos[s0:s0 + seg.length, 1] = s0 + r
                pos[s0:s0 + seg.length, 2] = s0 + c
        s0 += seg.length
    return np.broadcast_to(pos, (w.batch, S, A)).copy()


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray            # float32 [B][S][Hq][d]: exact values both sides consume
    k: np.ndarray            # float32 [B][S][Hkv][d]
    v: np.ndarray            # float32 [B][S][Hkv][d]
    q_bits: Optional[np.ndarray]  # uint16 bf16 patterns (bf16 workloads), else None
    k_bits: Optional[np.ndarray]
    v_bits: Optional[np.ndarray]
    w_q: Optional[np.ndarray]     # float32 [d] or None
    w_k: Optional[np.ndarray]
    positions: np.ndarray    # int32 [B][S][A]
    segments: np.ndarray     # int32 [B][nseg][3]


def _draw(rng, shape, bf16):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if not bf16:
        return x, None
    bits = f32_to_bf16_bits(x)
    return bf16_bits_to_f32(bits).reshape(shape), bits.reshape(shape)


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, S, Hq, Hkv, d = w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim
    bf16 = w.dtype == "bf16"
    q, qb = _draw(rng, (B, S, Hq, d), bf16)
    k, kb = _draw(rng, (B, S, Hkv, d), bf16)
    v, vb = _draw(rng, (B, S, Hkv, d), bf16)
    w_q = w_k = None
    if w.qk_norm:
        w_q = (1.0 + 0.02 * rng.standard_normal(size=(d,), dtype=np.float32)).astype(np.float32)
        w_k = (1.0 + 0.02 * rng.standard_normal(size=(d,), dtype=np.float32)).astype(np.float32)
    return Inputs(workload=w, q=q, k=k, v=v, q_bits=qb, k_bits=kb, v_bits=vb, w_q=w_q, w_k=w_k,
                  positions=positions_for(w), segments=segment_table(w))


@dataclass
class ProjectionInputs:
    """Inputs of the QKV projection in front of the path: the layer's hidden states and the
    fused q/k/v weight, both bf16 values (float32 arrays holding them, plus the patterns)."""
    x: np.ndarray        # float32 [B][S][hidden]
    x_bits: np.ndarray   # uint16
    w_qkv: np.ndarray    # float32 [(Hq + 2 Hkv) d][hidden]
    w_bits: np.ndarray   # uint16


def generate_projection(w: Workload, hidden: int, seed: Optional[int] = None) -> ProjectionInputs:
    """x ~ N(0, 1) and W ~ N(0, 1/hidden) (so each projected value is about N(0, 1)), drawn
    in that order from their own stream and rounded to bf16."""
    rng = np.random.Generator(np.random.PCG64(1000 + (w.seed if seed is None else seed)))
    n_out = (w.n_q_heads + 2 * w.n_kv_heads) * w.head_dim
    x, xb = _draw(rng, (w.batch, w.seq_len, hidden), True)
    wd = rng.standard_normal(size=(n_out, hidden), dtype=np.float32) * np.float32(1.0 / np.sqrt(hidden))
    wb = f32_to_bf16_bits(wd)
    return ProjectionInputs(x=x, x_bits=xb, w_qkv=bf16_bits_to_f32(wb).reshape(wd.shape),
                            w_bits=wb.reshape(wd.shape))
