"""Backward pass of the path in float64: gradients of a scalar loss, given d(loss)/d(out).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages train these models end to end with flow-matching and language-modelling losses
(HiDream-O1 atlas page, "How it works"; HunyuanImage 3.0 digest, training stages) but print
no backward formulas. What is here is the derivative of the forward in masked_attention.py,
norm.py and rope.py, written out with the chain rule:

Attention, for batch item b, query head h, KV head g = h // (Hq / Hkv) and mask M:
    Z = scale Q K^T (masked entries -inf),  P = softmax_rows(Z),  O = P V
    dV_g  = sum over the query heads h of group g of  P_h^T dO_h
    dP_h  = dO_h V_g^T
    dZ_h  = P_h * (dP_h - delta_h),   delta_h[i] = sum_j P_h[i, j] dP_h[i, j] = dO_h[i] . O_h[i]
    dQ_h  = scale dZ_h K_g,           dK_g = scale * sum over h of dZ_h^T Q_h
Rotary: each pair is rotated by an angle, an orthogonal map, so the gradient of its input
is the output gradient rotated by minus that angle.
RMSNorm: y = x r w with r = (mean(x^2) + eps)^(-1/2) over the head dim; with u = dy * w,
    dx = r u - x r^3 mean(x u),        dw = sum over tokens and heads of dy * x r

The row log-sum-exp lse[i] = log sum_j exp(Z[i, j]) over the allowed keys is what a
training forward keeps for the backward: with it, P = exp(Z - lse) needs no second
normalisation.
"""
from __future__ import annotations

import numpy as np

from .mask import explicit_mask
from .norm import rms_norm
from .rope import apply_rope, axis_of_pair, inv_freq, rope_angles


def _scores(Q, K, M, scale):
    return np.where(M, (Q @ K.T) * scale, -np.inf)


def _softmax(Z):
    m = np.max(Z, axis=-1, keepdims=True)
    e = np.exp(Z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_lse(q, k, masks, scale=None):
    """lse [B][Hq][S]: natural log of sum_j exp(scale q_i . k_j) over row i's allowed keys."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, S, Hq, d = q.shape
    group = Hq // k.shape[2]
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    lse = np.empty((B, Hq, S))
    for b in range(B):
        for h in range(Hq):
            Z = _scores(q[b, :, h], k[b, :, h // group], masks[b], scale)
            m = np.max(Z, axis=-1)
            lse[b, h] = m + np.log(np.sum(np.exp(Z - m[:, None]), axis=-1))
    return lse


def attention_backward(q, k, v, masks, dout, scale=None, groups=None):
    """(dq, dk, dv) of masked GQA attention, same layouts as q, k, v.

    groups: optional KV heads to compute (their query heads' dq and their dk, dv); the
    other entries are left as NaN."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    group = Hq // Hkv
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    groups = range(Hkv) if groups is None else groups
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    for b in range(B):
        for g in groups:
            K, V = k[b, :, g], v[b, :, g]
            dK = np.zeros((S, d))
            dV = np.zeros((S, d))
            for h in range(g * group, (g + 1) * group):
                Q, dO = q[b, :, h], dout[b, :, h]
                P = _softmax(_scores(Q, K, masks[b], scale))
                O = P @ V
                dV += P.T @ dO
                dP = dO @ V.T
                delta = np.sum(dO * O, axis=-1, keepdims=True)
                dZ = P * (dP - delta)
                dq[b, :, h] = scale * (dZ @ K)
                dK += scale * (dZ.T @ Q)
            dk[b, :, g] = dK
            dv[b, :, g] = dV
    return dq, dk, dv


def rope_backward(dy, angles):
    """Gradient of apply_rope's input: rotate every pair of dy by minus its angle."""
    return apply_rope(dy, -np.asarray(angles, dtype=np.float64))


def rms_norm_backward(x, weight, eps, dy):
    """(dx, dw) of rms_norm(x, weight, eps) for the output gradient dy.

    x, dy [..., d]; dw [d] is summed over every leading axis (tokens and heads)."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    u = dy * w
    dx = r * u - x * r ** 3 * np.mean(x * u, axis=-1, keepdims=True)
    dw = np.sum((dy * x * r).reshape(-1, x.shape[-1]), axis=0)
    return dx, dw


def _angles(w, positions):
    axes = axis_of_pair(w.rope, w.head_dim, w.mrope_sections)
    return rope_angles(positions, axes, inv_freq(w.rope_theta, w.head_dim))


def path_lse(inputs):
    """lse [B][Hq][S] of the whole path's attention (after the prologue)."""
    w = inputs.workload
    q, k = _prologue(inputs)[:2]
    masks = [explicit_mask(inputs.segments[b], w.seq_len) for b in range(w.batch)]
    return attention_lse(q, k, masks)


def _prologue(inputs):
    w = inputs.workload
    q = np.asarray(inputs.q, dtype=np.float64)
    k = np.asarray(inputs.k, dtype=np.float64)
    qn = rms_norm(q, inputs.w_q, w.norm_eps) if w.qk_norm else q
    kn = rms_norm(k, inputs.w_k, w.norm_eps) if w.qk_norm else k
    if w.rope == "none":
        return qn, kn, None
    ang = _angles(w, inputs.positions)
    return apply_rope(qn, ang), apply_rope(kn, ang), ang


def path_backward(inputs, dout, groups=None):
    """Gradients of the whole path (norm, rotary, mask, attention) for out gradient dout.

    Returns a dict: dq [B][S][Hq][d] and dk, dv [B][S][Hkv][d] with respect to the path's
    inputs q, k, v; dw_q, dw_k [d] with respect to the norm weights (None without q/k
    norm). groups: optional KV heads to compute; with it, dw_q and dw_k are not formed."""
    w = inputs.workload
    q = np.asarray(inputs.q, dtype=np.float64)
    k = np.asarray(inputs.k, dtype=np.float64)
    qr, kr, ang = _prologue(inputs)
    masks = [explicit_mask(inputs.segments[b], w.seq_len) for b in range(w.batch)]
    dqr, dkr, dv = attention_backward(qr, kr, inputs.v, masks, dout, groups=groups)
    dqn = dqr if ang is None else rope_backward(dqr, ang)
    dkn = dkr if ang is None else rope_backward(dkr, ang)
    out = {"dv": dv, "dw_q": None, "dw_k": None}
    if w.qk_norm:
        out["dq"], dwq = rms_norm_backward(q, inputs.w_q, w.norm_eps, dqn)
        out["dk"], dwk = rms_norm_backward(k, inputs.w_k, w.norm_eps, dkn)
        if groups is None:
            out["dw_q"], out["dw_k"] = dwq, dwk
    else:
        out["dq"], out["dk"] = dqn, dkn
    return out
