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

    # ---- training (bf16, Hq / Hkv in {1, 2, 4})
    def forward_train(self, q, k, v, stream=None):
        """(out, lse): the forward plus each row's log-sum-exp [B][Hq][S] for backward()."""
        out = torch.empty(self.shape, dtype=q.dtype, device=q.device)
        b, s, hq, _ = self.shape
        lse = torch.empty((b, hq, s), dtype=torch.float32, device=q.device)
        B.ha_attn_fwd_lse(self.desc, self.pro, q, k, v, out, lse, self.workspace, stream=stream)
        return out, lse

    def backward(self, q, k, v, out, lse, dout, stream=None):
        """(dq, dk, dv, dw_q, dw_k) for the output gradient dout; dw_* are None without
        q/k RMSNorm. The backward workspace is allocated on first use and kept."""
        if getattr(self, "bwd_workspace", None) is None:
            n = B.ha_attn_bwd_workspace_bytes(self.desc, self.pro)
            self.bwd_workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        norm = self.pro is not None and self.pro.c.q_norm_weight is not None
        dwq = torch.empty(self.shape[3], dtype=torch.float32, device=q.device) if norm else None
        dwk = torch.empty(self.shape[3], dtype=torch.float32, device=q.device) if norm else None
        B.ha_attn_bwd(self.desc, self.pro, q, k, v, out, lse, dout.contiguous(), dq, dk, dv, dwq, dwk,
                      self.bwd_workspace, stream=stream)
        return dq, dk, dv, dwq, dwk


class _HybridAttentionFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, attn, q, k, v, w_q, w_k):
        out, lse = attn.forward_train(q, k, v)
        ctx.attn = attn
        ctx.save_for_backward(q, k, v, out, lse)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse = ctx.saved_tensors
        dq, dk, dv, dwq, dwk = ctx.attn.backward(q, k, v, out, lse, dout.to(out.dtype))
        return None, dq, dk, dv, dwq, dwk


def hybrid_attention_train(attn: HybridAttention, q, k, v, w_q=None, w_k=None):
    """out = attn(q, k, v) recorded for torch autograd: out.backward() (or a loss built on it)
    fills q.grad, k.grad, v.grad and, when attn normalises q and k, the grads of the norm
    weight tensors w_q, w_k (the ones attn was built with)."""
    return _HybridAttentionFn.apply(attn, q, k, v, w_q, w_k)


def hybrid_attention(q, k, v, segments, **kw) -> torch.Tensor:
    b, s, hq, d = q.shape
    return HybridAttention(b, s, hq, k.shape[2], d, _dtype_name(q), segments,
                           device=q.device, **kw)(q, k, v)
