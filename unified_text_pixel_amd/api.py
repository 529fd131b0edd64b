"""Torch-facing convenience layer over the C ABI.

PyTorch only allocates the output, the workspace and the rotary table on the device and
supplies the stream; all computation runs in libha.so's kernels (binding.py)."""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import binding as B


def rope_table(theta: float, head_dim: int, n_pos: int, device="cuda") -> torch.Tensor:
    """(cos, sin) table float32 [n_pos][head_dim/2][2] on the device (fp64 host math)."""
    return torch.from_numpy(B.ha_rope_table_fill(theta, head_dim, n_pos)).to(device)


def _dtype_name(t: torch.Tensor) -> str:
    if t.dtype == torch.bfloat16:
        return "bf16"
    if t.dtype == torch.float32:
        return "f32"
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


class HybridAttention:
    """One layout (segment table, shapes, rotary and norm settings) with its workspace.

    q [B][S][Hq][d], k/v [B][S][Hkv][d] contiguous bf16 or fp32 on the GPU. segments:
    int [B][n_seg][3] rows of (start, length, kind) with kind 0 causal, 1 full, 2 image
    (generalized causal). rope: 'none', '1d', '2d' or 'mrope'; positions int32
    [B][S][n_axes] on the GPU."""

    def __init__(self, batch, seq_len, n_q_heads, n_kv_heads, head_dim, dtype, segments,
                 rope="none", positions=None, theta=1e4, mrope_sections=(0, 0, 0),
                 q_norm_weight=None, k_norm_weight=None, eps=1e-6, scale=0.0, cos_sin=None,
                 device="cuda"):
        self.desc = B.AttnDesc(batch, seq_len, n_q_heads, n_kv_heads, head_dim, dtype, segments,
                               scale)
        self.shape = (batch, seq_len, n_q_heads, head_dim)
        self.pro = None
        prologue = rope != "none" or q_norm_weight is not None
        if prologue:
            if rope != "none" and cos_sin is None:
                cos_sin = rope_table(theta, head_dim, max(1, seq_len), device)
            n_pos = 0 if cos_sin is None else cos_sin.shape[0]
            self.pro = B.PrologueDesc(rope, positions, cos_sin, n_pos, q_norm_weight,
                                      k_norm_weight, eps, mrope_sections)
        nbytes = B.ha_attn_workspace_bytes(self.desc, self.pro)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)

    def __call__(self, q, k, v, out=None, stream=None):
        if out is None:
            out = torch.empty(self.shape, dtype=q.dtype, device=q.device)
        B.ha_attn_fwd(self.desc, self.pro, q, k, v, out, self.workspace, stream=stream)
        return out


def hybrid_attention(q, k, v, segments, **kw) -> torch.Tensor:
    b, s, hq, d = q.shape
    return HybridAttention(b, s, hq, k.shape[2], d, _dtype_name(q), segments,
                           device=q.device, **kw)(q, k, v)
