"""ha_attn_fwd captured in a HIP graph (HybridAttention.graphed): every replay, with the
program's own eager work and synchronisations between replays, equals the eager call on the
same inputs bit for bit, and the first replay matches the oracle. Layouts cover the planned
path, forced split parts (device-built plan table, partial results, merge), Gen Image tile
lists, and no prologue."""
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import compare, f64, require_gpu
from test_gpu_parity import SMALL
from unified_text_pixel_amd import api
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def attention_for(w: W.Workload, dev, split_parts=0) -> api.HybridAttention:
    cs = api.rope_table(w.rope_theta, w.head_dim, max(1, w.seq_len)) if w.rope != "none" else None
    return api.HybridAttention(
        w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, W.segment_table(w),
        rope=w.rope, positions=dev["positions"] if w.rope != "none" else None, cos_sin=cs,
        mrope_sections=w.mrope_sections, q_norm_weight=dev["w_q"] if w.qk_norm else None,
        k_norm_weight=dev["w_k"] if w.qk_norm else None, eps=w.norm_eps, split_parts=split_parts)


GEN_SMALL = W.Workload(
    name="gen_graph", description="", batch=2,
    segments=(W.Segment(W.SEG_CAUSAL, 40), W.Segment(W.SEG_GEN, 64, (8, 8)),
              W.Segment(W.SEG_CAUSAL, 30), W.Segment(W.SEG_GEN, 100, (10, 10)),
              W.Segment(W.SEG_CAUSAL, 9)),
    n_q_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16", rope="2d", rope_theta=1e4,
    mrope_sections=(24, 20, 20), qk_norm=False, norm_eps=1e-6, seed=23)

CASES = [("hd_small", 0), ("hd_small", 3), ("edit_small", 2), ("gca_small", 0), ("gqa_g8", 0),
         ("gen", 0), ("gen", 2)]


@pytest.mark.parametrize("name,parts", CASES)
def test_graph_replays_equal_eager(name, parts):
    w = GEN_SMALL if name == "gen" else SMALL[name]
    print(f"case {name}: split_parts {parts} S={w.seq_len}", flush=True)
    x = W.generate(w)
    dev = to_device(x)
    attn = attention_for(w, dev, parts)
    q, k, v = dev["q"].clone(), dev["k"].clone(), dev["v"].clone()
    replay, out = attn.graphed(q, k, v)
    torch.cuda.synchronize()
    replay()
    torch.cuda.synchronize()
    compare(f64(out), oracle.hot_path(x), w.dtype, f"{name} graph replay")
    gen = torch.Generator(device="cuda").manual_seed(11)
    for r in range(3):
        # eager work between the replays: new inputs written by ordinary kernels, a sync
        for t in (q, k, v):
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
        torch.cuda.synchronize()
        replay()
        torch.cuda.synchronize()
        ref = attn(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, parts, r, float((out.float() - ref.float()).abs().max()))


@pytest.mark.parametrize("name,group", [("hunyuan", 1), ("page1024", 5)])
def test_graph_full_size(name, group):
    """Full-size layouts in a graph: the HunyuanImage interleave (S = 6016), whose call takes
    the device-built split plan, partial results and merge on the device's CUs, and the
    page-exact 1024^2 shape, whose attention runs in slice workgroups. Every replay equals the
    eager call bit for bit; the first matches the oracle on one KV group's heads."""
    cfg = dict(W.CONFIGS)
    cfg.update(W.page_shape_configs())
    w = cfg[name]
    print(f"case {name} full size, KV group {group}", flush=True)
    x = W.generate(w)
    dev = to_device(x)
    attn = attention_for(w, dev)
    q, k, v = dev["q"].clone(), dev["k"].clone(), dev["v"].clone()
    replay, out = attn.graphed(q, k, v)
    torch.cuda.synchronize()
    replay()
    torch.cuda.synchronize()
    G = w.n_q_heads // w.n_kv_heads
    heads = list(range(group * G, (group + 1) * G))
    compare(f64(out)[:, :, heads], oracle.hot_path(x, heads=heads)[:, :, heads], w.dtype,
            f"{name} graph replay, KV group {group}")
    gen = torch.Generator(device="cuda").manual_seed(12)
    for r in range(3):
        for t in (q, k, v):
            t.copy_(torch.randn(t.shape, generator=gen, device="cuda").to(t.dtype))
        torch.cuda.synchronize()
        replay()
        torch.cuda.synchronize()
        ref = attn(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (name, r, float((out.float() - ref.float()).abs().max()))
