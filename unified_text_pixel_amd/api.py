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
    (generalized causal), 3 Gen Image. rope: 'none', '1d', '2d' or 'mrope'; positions int32
    [B][S][n_axes] on the GPU. split_parts and plan_cus override the forward's split planner
    (ha_attn_desc)."""

    def __init__(self, batch, seq_len, n_q_heads, n_kv_heads, head_dim, dtype, segments,
                 rope="none", positions=None, theta=1e4, mrope_sections=(0, 0, 0),
                 q_norm_weight=None, k_norm_weight=None, eps=1e-6, scale=0.0, cos_sin=None,
                 device="cuda", split_parts=0, plan_cus=0):
        self.desc = B.AttnDesc(batch, seq_len, n_q_heads, n_kv_heads, head_dim, dtype, segments,
                               scale, split_parts=split_parts, plan_cus=plan_cus)
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
        self._args = (batch, seq_len, n_q_heads, n_kv_heads, head_dim, dtype, segments, scale)
        self._pro_args = (rope, positions, cos_sin, q_norm_weight, k_norm_weight, eps, mrope_sections)
        self._steps = None

    def __call__(self, q, k, v, out=None, stream=None):
        if out is None:
            out = torch.empty(self.shape, dtype=q.dtype, device=q.device)
        B.ha_attn_fwd(self.desc, self.pro, q, k, v, out, self.workspace, stream=stream)
        return out

    def graphed(self, q, k, v):
        """(replay, out): one forward on these q, k, v buffers captured in a HIP graph.
        replay() reruns the whole call (classifier, split plan, prologue, attention, merge)
        on the buffers' current contents with one graph launch on the current stream, writing
        out. The library allocates nothing, synchronises nothing and records no memory sets
        inside ha_attn_fwd, so the graph replays what was captured; its launches use this
        object's workspace, so replays and eager calls of one object must not overlap."""
        out = torch.empty(self.shape, dtype=q.dtype, device=q.device)
        side = torch.cuda.Stream(device=q.device)  # default priority
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self(q, k, v, out)  # outside the capture: the library's one-time device queries
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self(q, k, v, out)
        return graph.replay, out

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


    # ---- denoising steps over a step-invariant causal prefix
    def forward_from(self, q, k, v, begin, stream=None):
        """The forward of (q, k, v), recomputing only what tokens >= begin can change: the
        prologue from token begin on and the attention rows from begin on, over buffers kept
        in this object (rotated q and k, tile plan, output). The first call, or begin == 0,
        runs the whole path. Later calls are exact when the q, k, v rows below begin are the
        ones the previous call saw and no row below begin attends to a later token
        (prefix_is_invariant; a causal text prefix qualifies), which is checked. Returns the kept output
        tensor (overwritten by the next call)."""
        if not 0 <= begin <= self.shape[1]:
            raise ValueError(f"begin {begin} outside [0, {self.shape[1]}]")
        if not prefix_is_invariant(self.desc._seg_np, self.shape[1], begin):
            raise ValueError(f"rows below begin {begin} attend to later tokens: their outputs "
                             "would change with them")
        if self._steps is None:
            self._steps = self._plan(q)
            begin = 0
        st = self._steps
        if begin == 0:
            B.ha_classify_tiles(st["desc"], None, st["ranges"], st["lim"], stream)
        if st["pro"] is not None:
            B.ha_qk_prologue_from(st["desc"], st["pro"], q, k, st["qr"], st["kr"], begin, stream)
            qr, kr = st["qr"], st["kr"]
        else:
            qr, kr = q, k
        B.ha_attn_fwd_planned_from(st["desc"], qr, kr, v, st["lim"], st["ranges"], st["out"], begin,
                                   stream)
        return st["out"]

    def _plan(self, q):
        batch, seq_len, hq, hkv, d, dtype, segments, scale = self._args
        rope, positions, cos_sin, wq, wk, eps, sections = self._pro_args
        st = {"pro": None}
        if self.pro is not None:
            # the prologue writes q scaled by softmax scale * log2(e), taken as is by attention
            st["desc"] = B.AttnDesc(batch, seq_len, hq, hkv, d, dtype, segments, scale, q_prescaled=1)
            cs = self.pro._keep[1]
            st["pro"] = B.PrologueDesc(rope, positions, cs, 0 if cs is None else cs.shape[0], wq, wk,
                                       eps, sections, q_out_scale=B.ha_q_prescale(st["desc"]))
            st["qr"] = torch.empty(self.shape, dtype=q.dtype, device=q.device)
            st["kr"] = torch.empty((batch, seq_len, hkv, d), dtype=q.dtype, device=q.device)
        else:
            st["desc"] = self.desc
        _, _, nq, _ = B.ha_tile_shape(st["desc"])
        st["ranges"] = torch.empty((batch, nq, 2), dtype=torch.int32, device=q.device)
        st["lim"] = torch.empty((batch, seq_len), dtype=torch.int32, device=q.device)
        st["out"] = torch.empty(self.shape, dtype=q.dtype, device=q.device)
        return st


def prefix_is_invariant(segments, seq_len: int, p: int) -> bool:
    """True when no query row below p attends to a key at or after p, in any batch item of
    a segment table [B][n_seg][3] (start, length, kind: 0 causal, 1 full, 2 image, 3 Gen
    Image): rows below p then give the same output whatever tokens >= p hold. A causal row i
    sees keys <= i, so causal segments never break it; a full segment's rows see every key,
    so one that starts below p < seq_len does; an image segment's rows (GCA or Gen Image) see
    keys below its end, so one that p splits does. ha_attn_fwd_planned_from makes the same
    check and refuses a row_begin that fails it."""
    if not 0 <= p <= seq_len:
        return False
    seg = np.asarray(segments, dtype=np.int64).reshape(-1, 3)
    for st, ln, kind in seg:
        if ln <= 0:
            continue
        if kind == 1 and st < p < seq_len:
            return False
        if kind in (2, 3) and st < p < st + ln:
            return False
    return True


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
