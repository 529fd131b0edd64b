"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI on seeded
inputs, and compare with the oracle at the stated tolerances."""
from __future__ import annotations

import contextlib
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from unified_text_pixel_amd import api, binding as B
from workloads.device import to_device

# Tolerances: bf16 inputs, max |err| <= 2e-2 and mean |err| <= 2e-3 against the oracle;
# fp32 inputs, max |err| <= 1e-5 * max |oracle| over the whole output.
BF16_MAX, BF16_MEAN, F32_REL = 2e-2, 2e-3, 1e-5


_PLAN = {"split_parts": 0, "plan_cus": 0}


@contextlib.contextmanager
def plan(split_parts=0, plan_cus=0):
    """Descriptors made by desc_for inside the block carry these split-plan overrides
    (ha_attn_desc.split_parts: 1 never splits, P > 1 splits every query block into P parts;
    plan_cus: plan for that many CUs instead of the device's)."""
    old = dict(_PLAN)
    _PLAN.update(split_parts=int(split_parts), plan_cus=int(plan_cus or 0))
    try:
        yield
    finally:
        _PLAN.update(old)


def unsplit():
    """The bf16 forward without split query blocks: one work item per query block, the
    summation order of ha_attn_fwd_planned."""
    return plan(split_parts=1)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def desc_for(w: W.Workload, segments=None) -> B.AttnDesc:
    seg = W.segment_table(w) if segments is None else segments
    return B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, seg,
                      split_parts=_PLAN["split_parts"], plan_cus=_PLAN["plan_cus"])


def prologue_for(w: W.Workload, dev) -> B.PrologueDesc | None:
    if w.rope == "none" and not w.qk_norm:
        return None
    cs = api.rope_table(w.rope_theta, w.head_dim, max(1, w.seq_len)) if w.rope != "none" else None
    return B.PrologueDesc(w.rope, dev["positions"] if w.rope != "none" else None, cs,
                          0 if cs is None else cs.shape[0], dev["w_q"], dev["w_k"], w.norm_eps,
                          w.mrope_sections)


def run_fwd(inputs, dev=None, segments=None):
    """Whole path through ha_attn_fwd; returns (out tensor, device dict)."""
    w = inputs.workload
    dev = to_device(inputs) if dev is None else dev
    desc = desc_for(w, segments if segments is not None else inputs.segments)
    pro = prologue_for(w, dev)
    ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, pro)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(dev["q"])
    B.ha_attn_fwd(desc, pro, dev["q"], dev["k"], dev["v"], out, ws)
    torch.cuda.synchronize()
    return out, dev


def refresh_bits(x):
    """After editing x.q / x.k / x.v in fp32: round them to bf16 again (bf16 workloads), so
    the device copy and the oracle see the same values."""
    if x.workload.dtype == "bf16":
        for n in ("q", "k", "v"):
            bits = W.f32_to_bf16_bits(getattr(x, n))
            setattr(x, n + "_bits", bits.reshape(getattr(x, n).shape))
            setattr(x, n, W.bf16_bits_to_f32(bits).reshape(getattr(x, n).shape))
    return x


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    err = np.abs(got - want)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "bf16":
        mx, mean = float(err.max()), float(err.mean())
        print(f"{what}: max|err| {mx:.3e} mean|err| {mean:.3e}", flush=True)
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (what, mx, mean)
    else:
        rel = float(err.max() / np.abs(want).max())
        print(f"{what}: max|err|/max|ref| {rel:.3e}", flush=True)
        assert rel <= F32_REL, (what, rel)


def sample_rows(w: W.Workload, n_random=40, seed=0):
    S = w.seq_len
    rows = {0, 1, 2, 3, S - 1, S - 2}
    at = 0
    for s in w.segments:
        rows.update({at, at + 1, at + s.length - 1, at + s.length - 2})
        at += s.length
    for t in (31, 32, 63, 64, 65, 127, 128):
        rows.add(t)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, S, size=n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < S))
