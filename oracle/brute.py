"""Scalar pure-Python float64 re-derivation of the whole path, for tiny inputs only.

Written independently of the vectorised oracle (scalar loops over every index, the math
module's sqrt/cos/sin/exp, segment membership recomputed from the table for every pair)
so that the two can check each other. Same readings as the rest of the oracle:
  RMSNorm  y = x / sqrt(mean(x^2) + eps) * w          (model card, "q/k RMSNorm")
  rotary   pair (i, i + d/2) rotated by pos[axis(i)] * base^(-2i/d); axis(i) deals the
           pairs to the axes in turn within each axis's section count
           (HunyuanImage 3.0 digest, generalized 2D RoPE; model card, mRoPE [24,20,20])
  mask     causal j <= i; full always; image segment j <= i or same segment; never a
           key of a Gen Image (multi-image training) that ended at or before i
           (HiDream-O1 atlas page, "How it works"; HunyuanImage 3.0 digest,
           "Generalized Causal Attention" and its multi-generation training paragraph)
  softmax  over allowed keys of scale * q.k, scale = 1/sqrt(d)
"""
from __future__ import annotations

import math


def _axis_list(kind, half, sections):
    if kind in ("none", "1d"):
        return [0] * half
    if kind == "2d":
        return [i % 2 for i in range(half)]
    order = []
    for rnd in range(max(sections)):
        for a in range(3):
            if rnd < sections[a]:
                order.append(a)
    return order


def _kind_and_segment(table, t):
    for idx, row in enumerate(table):
        start, length, kind = int(row[0]), int(row[1]), int(row[2])
        if start <= t < start + length:
            return kind, idx
    raise ValueError("token outside the segment table")


def _allowed(table, i, j):
    kind_j, seg_j = _kind_and_segment(table, j)
    if kind_j == 3 and i >= int(table[seg_j][0]) + int(table[seg_j][1]):
        return False  # key in a Gen Image that token i comes after
    kind_i, seg_i = _kind_and_segment(table, i)
    if kind_i == 0:
        return j <= i
    if kind_i == 1:
        return True
    return j <= i or seg_j == seg_i


def _prep(vec, w, weight, pos, axes):
    d = len(vec)
    x = [float(t) for t in vec]
    if w.qk_norm:
        ss = 0.0
        for t in x:
            ss += t * t
        r = 1.0 / math.sqrt(ss / d + w.norm_eps)
        x = [x[e] * r * float(weight[e]) for e in range(d)]
    if w.rope == "none":
        return x
    half = d // 2
    y = list(x)
    for i in range(half):
        ang = float(pos[axes[i]]) * math.pow(w.rope_theta, -2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        y[i] = x[i] * c - x[i + half] * s
        y[i + half] = x[i + half] * c + x[i] * s
    return y


def brute_force(inputs):
    """Nested lists out[b][i][h][e] of the whole path, float64 scalars."""
    w = inputs.workload
    B, S, Hq, Hkv, d = w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim
    axes = _axis_list(w.rope, d // 2, w.mrope_sections)
    scale = 1.0 / math.sqrt(d)
    out = []
    for b in range(B):
        table = inputs.segments[b]
        pos = inputs.positions[b]
        qs = [[_prep(inputs.q[b][i][h], w, inputs.w_q, pos[i], axes) for h in range(Hq)]
              for i in range(S)]
        ks = [[_prep(inputs.k[b][j][g], w, inputs.w_k, pos[j], axes) for g in range(Hkv)]
              for j in range(S)]
        ob = []
        for i in range(S):
            oi = []
            for h in range(Hq):
                g = h * Hkv // Hq
                scores = []
                for j in range(S):
                    if _allowed(table, i, j):
                        dot = 0.0
                        for e in range(d):
                            dot += qs[i][h][e] * ks[j][g][e]
                        scores.append((j, dot * scale))
                top = max(s for _, s in scores)
                wsum = 0.0
                acc = [0.0] * d
                for j, s in scores:
                    p = math.exp(s - top)
                    wsum += p
                    vj = inputs.v[b][j][g]
                    for e in range(d):
                        acc[e] += p * float(vj[e])
                oi.append([a / wsum for a in acc])
            ob.append(oi)
        out.append(ob)
    return out
