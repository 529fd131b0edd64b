"""q/k RMSNorm over the head dimension.

hidream-o1-p100a model card, architecture paragraph: the backbone applies RMSNorm to q
and k ("q/k RMSNorm"). The page gives no formula; the reading used here is the standard
RMSNorm: y = x / sqrt(mean(x^2) + eps) * w, eps inside the square root, one weight
vector of length head_dim shared by all heads, applied before the rotary embedding.
"""
from __future__ import annotations

import numpy as np


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float, dtype=np.float64) -> np.ndarray:
    x = np.asarray(x, dtype=dtype)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + dtype(eps)) * np.asarray(weight, dtype=dtype)
