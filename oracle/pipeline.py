"""The whole path in the pages' order: q/k RMSNorm, rotary embedding, mask, attention.

Order: norm then rotary on q and k (never on v), as in a Qwen3-style block with q/k
RMSNorm (hidream-o1-p100a model card, architecture paragraph); then masked attention
(mask.py, masked_attention.py). Workloads without q/k norm (the HunyuanImage layout and the tiny
fp32 check) skip that step; rotary kind "none" skips the rotation.
"""
from __future__ import annotations

import numpy as np

from .masked_attention import attention, attention_rows
from .mask import explicit_mask, mask_rows
from .norm import rms_norm
from .rope import apply_rope, axis_of_pair, inv_freq, rope_angles


def _rotary(x, workload, positions, dtype):
    if workload.rope == "none":
        return np.asarray(x, dtype=dtype)
    axes = axis_of_pair(workload.rope, workload.head_dim, workload.mrope_sections)
    ang = rope_angles(positions, axes, inv_freq(workload.rope_theta, workload.head_dim))
    return apply_rope(x, ang, dtype=dtype)


def prologue(inputs, dtype=np.float64):
    """Normalised and rotated (q, k), same layouts as the inputs."""
    w = inputs.workload
    q = np.asarray(inputs.q, dtype=dtype)
    k = np.asarray(inputs.k, dtype=dtype)
    if w.qk_norm:
        q = rms_norm(q, inputs.w_q, w.norm_eps, dtype=dtype)
        k = rms_norm(k, inputs.w_k, w.norm_eps, dtype=dtype)
    return _rotary(q, w, inputs.positions, dtype), _rotary(k, w, inputs.positions, dtype)


def hot_path(inputs, dtype=np.float64, heads=None):
    """out [B][S][Hq][d] of the whole path; optionally only some query heads."""
    w = inputs.workload
    q, k = prologue(inputs, dtype)
    masks = [explicit_mask(inputs.segments[b], w.seq_len) for b in range(w.batch)]
    return attention(q, k, inputs.v, masks, dtype=dtype, heads=heads)


def hot_path_rows(inputs, b, rows, heads, dtype=np.float64):
    """Selected outputs [len(rows)][len(heads)][d] of batch item b, computing the prologue
    only where it is needed (sampled q rows, every k row of item b)."""
    w = inputs.workload
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(inputs.q[b:b + 1, rows], dtype=dtype)
    k = np.asarray(inputs.k[b:b + 1], dtype=dtype)
    if w.qk_norm:
        q = rms_norm(q, inputs.w_q, w.norm_eps, dtype=dtype)
        k = rms_norm(k, inputs.w_k, w.norm_eps, dtype=dtype)
    q = _rotary(q, w, inputs.positions[b:b + 1, rows], dtype)[0]
    k = _rotary(k, w, inputs.positions[b:b + 1], dtype)[0]
    mrows = mask_rows(inputs.segments[b], w.seq_len, rows)
    # attention_rows indexes q by token; q here is already restricted to `rows`.
    return attention_rows(q, k, inputs.v[b], mrows, np.arange(len(rows)), heads, dtype=dtype)
