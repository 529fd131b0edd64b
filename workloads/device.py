"""Move generated inputs to a torch device (bf16 tensors are built from the exact 16-bit
patterns the generator rounded to). Marshalling only."""
from __future__ import annotations

import numpy as np
import torch


def _t(bits_or_f32, bf16, device):
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(bits_or_f32).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(bits_or_f32, dtype=np.float32)).to(device)


def to_device(inputs, device="cuda"):
    """dict of device tensors: q, k, v, positions, w_q, w_k (None when absent)."""
    bf16 = inputs.workload.dtype == "bf16"
    d = {
        "q": _t(inputs.q_bits if bf16 else inputs.q, bf16, device),
        "k": _t(inputs.k_bits if bf16 else inputs.k, bf16, device),
        "v": _t(inputs.v_bits if bf16 else inputs.v, bf16, device),
        "positions": torch.from_numpy(np.ascontiguousarray(inputs.positions)).to(device),
        "w_q": None if inputs.w_q is None else torch.from_numpy(inputs.w_q).to(device),
        "w_k": None if inputs.w_k is None else torch.from_numpy(inputs.w_k).to(device),
    }
    return d


def projection_to_device(p, device="cuda"):
    """(x, w_qkv) as bf16 device tensors."""
    return _t(p.x_bits, True, device), _t(p.w_bits, True, device)
