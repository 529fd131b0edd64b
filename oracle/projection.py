"""QKV projection followed by the q/k prologue, as one operation.

TEST INFRASTRUCTURE ONLY (see the package docstring).

In each backbone layer q, k and v come from the layer's normalised hidden states through one
linear map, and q and k then go through RMSNorm and the rotary embedding before attention
(hidream-o1-p100a model card, "What this model is": the Qwen3-VL-8B language model, hidden
size 4096, GQA 32/8, head dim 128, q/k RMSNorm, mRoPE). Readings, the pages printing no
layout: the weight is in the linear-layer layout W [(Hq + 2 Hkv) d][hidden], its rows the
q heads, then the k heads, then the v heads, each head's d rows in order; y = x W^T with
no bias (none is stated). Nothing is rounded between the product and the prologue.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .pipeline import prologue


def qkv_projection(x, w_qkv, n_q_heads, n_kv_heads, head_dim, dtype=np.float64):
    """(q, k, v) = x W^T split by heads: x [B][S][hidden] -> q [B][S][Hq][d],
    k and v [B][S][Hkv][d]."""
    x = np.asarray(x, dtype=dtype)
    w = np.asarray(w_qkv, dtype=dtype)
    B, S, _ = x.shape
    y = x @ w.T
    nq, nkv = n_q_heads * head_dim, n_kv_heads * head_dim
    q = y[..., :nq].reshape(B, S, n_q_heads, head_dim)
    k = y[..., nq:nq + nkv].reshape(B, S, n_kv_heads, head_dim)
    v = y[..., nq + nkv:nq + 2 * nkv].reshape(B, S, n_kv_heads, head_dim)
    return q, k, v


def qkv_prologue(inputs, x, w_qkv, dtype=np.float64):
    """(q_rot, k_rot, v): the projection of x, then q/k RMSNorm and rotary as the path's
    prologue applies them (norm weights, positions and rotary settings from inputs)."""
    w = inputs.workload
    q, k, v = qkv_projection(x, w_qkv, w.n_q_heads, w.n_kv_heads, w.head_dim, dtype)
    q_rot, k_rot = prologue(dataclasses.replace(inputs, q=q, k=k, v=v), dtype)
    return q_rot, k_rot, v
