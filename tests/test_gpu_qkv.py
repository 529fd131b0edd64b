"""The QKV projection with the prologue in its epilogue (ha_qkv_prologue) against the
oracle's projection + prologue, through the C ABI.

Tolerance: the product accumulates bf16 x bf16 terms in fp32 (relative error about
hidden * 2^-24, far below bf16), the norm and rotary run in fp32, and each output is
rounded once to bf16 (relative 2^-9): |got - want| <= 2^-8 |want| + ABS."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import compare, f64, require_gpu
from unified_text_pixel_amd import api, binding as B
from workloads.device import projection_to_device, to_device

pytestmark = pytest.mark.gpu
C, F, G = W.SEG_CAUSAL, W.SEG_FULL, W.SEG_GCA
ABS = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def layout(segs, hq=8, hkv=2, rope="mrope", norm=True, batch=2, theta=5e6, seed=51):
    return W.Workload(name="qkv", description="", batch=batch, segments=tuple(segs), n_q_heads=hq,
                      n_kv_heads=hkv, head_dim=128, dtype="bf16", rope=rope, rope_theta=theta,
                      mrope_sections=(24, 20, 20), qk_norm=norm, norm_eps=1e-6, seed=seed)


def run_qkv(w, x_in, proj, prescale=False, with_pro=True):
    dev = to_device(x_in)
    xd, wd = projection_to_device(proj)
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, 128, "bf16", x_in.segments)
    pro = None
    if with_pro:
        cs = api.rope_table(w.rope_theta, 128, w.seq_len) if w.rope != "none" else None
        pro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0], dev["w_q"],
                             dev["w_k"], w.norm_eps, w.mrope_sections,
                             q_out_scale=B.ha_q_prescale(desc) if prescale else 0.0)
    q = torch.empty((w.batch, w.seq_len, w.n_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((w.batch, w.seq_len, w.n_kv_heads, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    B.ha_qkv_prologue(desc, pro, xd, proj.x.shape[-1], wd, q, k, v)
    torch.cuda.synchronize()
    return q, k, v, desc, dev


def check(name, got, want):
    err = np.abs(got - want)
    bad = err > 2.0 ** -8 * np.abs(want) + ABS
    print(f"{name}: max|err| {err.max():.3e} worst rel {(err / (np.abs(want) + ABS)).max():.3e}", flush=True)
    assert not bad.any(), (name, int(bad.sum()))


CASES = {
    # rows not a multiple of the 256-token tile, mRoPE + norm, 12 heads (6 feature tiles)
    "mrope_norm": (layout([W.Segment(C, 70), W.Segment(F, 64, (8, 8))]), 256),
    # one stage of 64, 2D rotary without norm
    "one_stage_2d": (layout([W.Segment(C, 20), W.Segment(G, 49, (7, 7))], rope="2d", norm=False, theta=1e4), 64),
    # odd stage count (the tail stage), 1D rotary
    "odd_stages": (layout([W.Segment(C, 300)], rope="1d", batch=1), 192),
    # an odd number of heads (3): the second wave of the last feature tile has no head
    "odd_heads": (layout([W.Segment(C, 40), W.Segment(F, 100, (10, 10))], hq=1, hkv=1), 128),
    # several token tiles and feature tiles, GQA 32/8, tokens not a tile multiple
    "gqa_32_8": (layout([W.Segment(C, 258), W.Segment(F, 1024, (32, 32))], hq=32, hkv=8, batch=1), 320),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("prescale", [False, True])
def test_qkv_prologue_parity(name, prescale):
    w, hidden = CASES[name]
    x_in = W.generate(w)
    proj = W.generate_projection(w, hidden)
    q, k, v, desc, _ = run_qkv(w, x_in, proj, prescale)
    q_ref, k_ref, v_ref = oracle.qkv_prologue(x_in, proj.x, proj.w_qkv)
    if prescale:
        q_ref = q_ref * float(np.float32(B.ha_q_prescale(desc)))
    check(f"{name} q", f64(q), q_ref)
    check(f"{name} k", f64(k), k_ref)
    check(f"{name} v", f64(v), v_ref)


def test_plain_projection_without_prologue():
    w, hidden = CASES["mrope_norm"]
    x_in = W.generate(w)
    proj = W.generate_projection(w, hidden)
    q, k, v, _, _ = run_qkv(w, x_in, proj, with_pro=False)
    q_ref, k_ref, v_ref = oracle.qkv_projection(proj.x, proj.w_qkv, w.n_q_heads, w.n_kv_heads, 128)
    for n, got, want in (("q", q, q_ref), ("k", k, k_ref), ("v", v, v_ref)):
        check(f"plain {n}", f64(got), want)


@pytest.mark.parametrize("name", ["hd2048", "hunyuan"])
def test_full_size_sampled_tokens(name):
    """A full layer, hidden 4096, GQA 32/8 (6144 outputs per token), in the benchmark's launch
    configuration: the hd2048 layer (2 x 4354 tokens, RMSNorm + mRoPE) and the HunyuanImage
    layer (6016 tokens, 2D rotary on images and 1D on text, no norm; a different split between
    the main tiles and the tail); sampled tokens of every batch item (both ends, the edges of
    the main and tail tiles, random ones) against the oracle."""
    w = W.get_config(name)
    x_in = W.generate(w)
    proj = W.generate_projection(w, 4096)
    q, k, v, desc, _ = run_qkv(w, x_in, proj, prescale=True)
    scale = float(np.float32(B.ha_q_prescale(desc)))
    rng = np.random.default_rng(3)
    S = w.seq_len
    for b in range(w.batch):
        rows = np.unique(np.r_[0, 1, 255, 256, 257, 5375, 5376, 5377, S - 1,
                               rng.integers(0, S, 40)])
        rows = rows[rows < S]
        sub = dataclasses.replace(x_in, workload=w.replace(batch=1), q=x_in.q[b:b + 1, rows],
                                  k=x_in.k[b:b + 1, rows], v=x_in.v[b:b + 1, rows],
                                  positions=x_in.positions[b:b + 1, rows], segments=x_in.segments[b:b + 1])
        q_ref, k_ref, v_ref = oracle.qkv_prologue(sub, proj.x[b:b + 1, rows], proj.w_qkv)
        check(f"{name} item {b} q", f64(q[b, rows]), q_ref[0] * scale)
        check(f"{name} item {b} k", f64(k[b, rows]), k_ref[0])
        check(f"{name} item {b} v", f64(v[b, rows]), v_ref[0])


def test_feeds_attention():
    """ha_qkv_prologue (q prescaled) straight into ha_attn_fwd_planned equals the oracle's
    whole path on the projected q, k, v."""
    w, hidden = CASES["mrope_norm"]
    x_in = W.generate(w)
    proj = W.generate_projection(w, hidden)
    q, k, v, _, dev = run_qkv(w, x_in, proj, prescale=True)
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, 128, "bf16", x_in.segments, q_prescaled=1)
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    ranges = torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda")
    lim = torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")
    B.ha_classify_tiles(desc, None, ranges, lim)
    out = torch.empty_like(q)
    B.ha_attn_fwd_planned(desc, q, k, v, lim, ranges, out)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref = oracle.qkv_prologue(x_in, proj.x, proj.w_qkv)
    masks = [oracle.explicit_mask(x_in.segments[b], w.seq_len) for b in range(w.batch)]
    compare(f64(out), oracle.attention(q_ref, k_ref, v_ref, masks), "bf16", "qkv -> attention")
