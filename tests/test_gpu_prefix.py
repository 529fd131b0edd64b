"""Step-invariant causal prefix: recomputing only the rows after it.

A causal prefix (text + markers at the front) never attends to what follows it, so across
denoising steps its prologue outputs and attention outputs stay the same; only the rows
after it need recomputing. Modelled here as two steps: step 0 runs the whole path; for step
1 the tokens after the prefix get new q, k, v, and only ha_qk_prologue_from and
ha_attn_fwd_planned_from run from the prefix end on the buffers step 0 left. The result must
equal, bit for bit, a whole-path run on the step-1 inputs with one work item per query block
(the same kernels over the same values; where ha_attn_fwd splits query blocks into parts, its
merge rounds differently), and match the oracle on the step-1 inputs within the bf16 gates."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import compare, f64, refresh_bits, require_gpu, run_fwd, unsplit
from unified_text_pixel_amd import api, binding as B
from workloads.device import to_device

pytestmark = pytest.mark.gpu
C, F = W.SEG_CAUSAL, W.SEG_FULL


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def hidream(text, grid, batch=2, seed=41):
    return W.Workload(name="prefix", description="", batch=batch,
                      segments=(W.Segment(C, text), W.Segment(F, grid * grid, (grid, grid))),
                      n_q_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16", rope="mrope",
                      rope_theta=5e6, mrope_sections=(24, 20, 20), qk_norm=True, seed=seed)


def two_steps(w, p, row_begin=None):
    """GPU out of step 1 computed from p on, the whole-path out of step 1, the oracle's."""
    row_begin = p if row_begin is None else row_begin
    x = W.generate(w)
    dev = to_device(x)
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, "bf16", x.segments,
                      q_prescaled=1)
    cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len)
    pro = B.PrologueDesc(w.rope, dev["positions"], cs, cs.shape[0], dev["w_q"], dev["w_k"], w.norm_eps,
                         w.mrope_sections, q_out_scale=B.ha_q_prescale(desc))
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    ranges = torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda")
    lim = torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")
    B.ha_classify_tiles(desc, None, ranges, lim)
    qr, kr, out = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["q"])
    # step 0: the whole path
    B.ha_qk_prologue(desc, pro, dev["q"], dev["k"], qr, kr)
    B.ha_attn_fwd_planned(desc, qr, kr, dev["v"], lim, ranges, out)
    torch.cuda.synchronize()
    # step 1: new q, k, v after the prefix (the denoiser's new hidden states there)
    rng = np.random.default_rng(99)
    for n in ("q", "k", "v"):
        a = getattr(x, n)
        a[:, p:] = rng.standard_normal(a[:, p:].shape).astype(np.float32)
    refresh_bits(x)
    dev1 = to_device(x)
    for n in ("q", "k", "v"):
        dev[n][:, p:] = dev1[n][:, p:]
    B.ha_qk_prologue_from(desc, pro, dev["q"], dev["k"], qr, kr, p)
    B.ha_attn_fwd_planned_from(desc, qr, kr, dev["v"], lim, ranges, out, row_begin)
    with unsplit():
        whole, _ = run_fwd(x, dev1)
    torch.cuda.synchronize()
    return out, whole, x


@pytest.mark.parametrize("text,grid,p", [(70, 16, 70), (258, 32, 258), (100, 12, 37)])
def test_prefix_step_equals_whole_path(text, grid, p):
    """p = the text length (prefix end inside or at a query block edge), and a p inside the
    text (its rows are causal too, so still exact)."""
    w = hidream(text, grid)
    print(f"case text={text} grid={grid}x{grid} p={p}", flush=True)
    out, whole, x = two_steps(w, p)
    assert torch.equal(out, whole), "prefix step differs from the whole path"
    compare(f64(out), oracle.hot_path(x), "bf16", f"prefix p={p}")


def test_row_begin_zero_is_the_planned_path():
    w = hidream(40, 10, batch=1)
    out, whole, x = two_steps(w, 0, row_begin=0)
    assert torch.equal(out, whole)


def test_rows_before_row_begin_untouched():
    """Rows below row_begin keep what the buffer held, even inside a computed block (row 100
    of the causal text lies inside the block of rows [86, 150), the sequence being 406 long
    with blocks of 64 aligned to its end)."""
    w = hidream(150, 16, batch=1, seed=43)
    x = W.generate(w)
    dev = to_device(x)
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, "bf16", x.segments)
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    ranges = torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda")
    lim = torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")
    B.ha_classify_tiles(desc, None, ranges, lim)
    out = torch.full_like(dev["q"], 7.0)
    assert (w.seq_len - 100) % bq != 0, "row 100 must sit inside a block"
    B.ha_attn_fwd_planned_from(desc, dev["q"], dev["k"], dev["v"], lim, ranges, out, 100)
    torch.cuda.synchronize()
    assert bool((out[:, :100] == 7.0).all())
    ref = torch.empty_like(dev["q"])
    B.ha_attn_fwd_planned(desc, dev["q"], dev["k"], dev["v"], lim, ranges, ref)
    torch.cuda.synchronize()
    assert torch.equal(out[:, 100:], ref[:, 100:])


@pytest.mark.parametrize("rope,norm", [("mrope", True), ("none", False)])
def test_api_forward_from_over_steps(rope, norm):
    """HybridAttention.forward_from over three denoising steps, each with new tokens after
    the text, equals the whole forward of that step's inputs (one work item per query
    block); begin inside the generation grid is refused."""
    w = hidream(66, 12, seed=47).replace(rope=rope, qk_norm=norm)
    x = W.generate(w)
    dev = to_device(x)
    attn = api.HybridAttention(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, "bf16",
                               x.segments, rope=w.rope, positions=dev["positions"], theta=w.rope_theta,
                               mrope_sections=w.mrope_sections,
                               q_norm_weight=dev["w_q"] if norm else None,
                               k_norm_weight=dev["w_k"] if norm else None, eps=w.norm_eps)
    whole = api.HybridAttention(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, "bf16",
                                x.segments, rope=w.rope, positions=dev["positions"], theta=w.rope_theta,
                                mrope_sections=w.mrope_sections,
                                q_norm_weight=dev["w_q"] if norm else None,
                                k_norm_weight=dev["w_k"] if norm else None, eps=w.norm_eps, split_parts=1)
    q, k, v = dev["q"].clone(), dev["k"].clone(), dev["v"].clone()
    gen = torch.Generator(device="cuda").manual_seed(3)
    for step in range(3):
        if step:
            for t in (q, k, v):
                t[:, 66:] = torch.randn(t[:, 66:].shape, generator=gen, device="cuda").to(t.dtype)
        got = attn.forward_from(q, k, v, 66 if step else 0)
        want = whole(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {step}"
    with pytest.raises(ValueError):
        attn.forward_from(q, k, v, 67)


def test_prefix_step_full_size_hd2048():
    """The 2048^2 layout at full size (2 x 4354 tokens, GQA 32/8): a step from the end of the
    258-token text prefix equals the whole path bit for bit, and sampled rows after the prefix
    match the oracle on the step-1 inputs."""
    w = W.get_config("hd2048")
    print("case hd2048 full size, p=258", flush=True)
    out, whole, x = two_steps(w, 258)
    assert torch.equal(out, whole), "prefix step differs from the whole path"
    got = f64(out)
    rng = np.random.default_rng(5)
    rows = np.unique(np.r_[258, 259, 321, 322, 4353, rng.integers(258, w.seq_len, 20)])
    for b in range(w.batch):
        want = oracle.hot_path_rows(x, b, rows, list(range(w.n_q_heads)))
        compare(got[b, rows], want, "bf16", f"hd2048 prefix step, item {b} ({len(rows)} rows x 32 heads)")
