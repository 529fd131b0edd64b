"""Training path against the oracle's gradients, through the C ABI.

ha_attn_fwd_lse, then ha_attn_bwd with a seeded bf16 output gradient; the oracle's
path_backward (fp64; pinned by finite differences, torch autograd and closed forms) is the
reference for dq, dk, dv and the norm-weight gradients, attention_lse for the lse.

Tolerance. Every product runs on bf16 operands (q', k, v, dO, and P or dZ rounded to bf16)
with fp32 accumulation, and dq, dk, dv are rounded to bf16: a gradient row (one token and
head over the head dim) is a sum of terms carrying two to four bf16 roundings (relative
2^-9 each), so its rms error is a few times 2^-9 of the row's own size. Row sizes differ by
an order of magnitude (a causal row near the start of the sequence, with few keys, has a
far larger dq than a full row), so the bound is per row. A row's rounding error follows the
size of its terms (P (dP - delta) k), not of their sum, which cancels in some rows (and is
exactly zero for dq of a row that sees one key), so each row is measured against the larger
of its own rms and ROW_FLOOR * rms of the whole tensor. The bulk of the rows (99%) must
stay within GRAD_ROW_BULK (a few roundings); any row within GRAD_ROW, which leaves room for
terms up to ~10x the row's floored size (3 roundings x 2^-9 x 10 ~ 6%); and mean |err| <=
GRAD_MEAN * rms over the tensor. A wrong tile or mask leaves errors the size of the row
itself. The norm-weight gradients are one row each. lse is the log of a sum of exponentials of
bf16-operand scores: |err| <= LSE_ABS."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import desc_for, f64, plan, prologue_for, require_gpu
from unified_text_pixel_amd import binding as B
from workloads.device import to_device

pytestmark = pytest.mark.gpu

C, F, G, GEN = W.SEG_CAUSAL, W.SEG_FULL, W.SEG_GCA, W.SEG_GEN
GRAD_ROW, GRAD_ROW_BULK, GRAD_MEAN, ROW_FLOOR, LSE_ABS = 5e-2, 1e-2, 1e-2, 0.5, 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def small(segs, hq=8, hkv=2, d=128, rope="mrope", norm=True, batch=2, theta=5e6, seed=31):
    sections = (24, 20, 20) if d == 128 else (12, 10, 10)
    return W.Workload(name="small", description="", batch=batch, segments=tuple(segs),
                      n_q_heads=hq, n_kv_heads=hkv, head_dim=d, dtype="bf16", rope=rope,
                      rope_theta=theta, mrope_sections=sections, qk_norm=norm, norm_eps=1e-6,
                      seed=seed)


SMALL = {
    "hd_small": small([W.Segment(C, 70), W.Segment(F, 256, (16, 16))]),
    "edit_small": small([W.Segment(C, 40), W.Segment(F, 100, (10, 10)), W.Segment(C, 81, (9, 9))]),
    "gca_small": small([W.Segment(C, 33), W.Segment(G, 64, (8, 8)), W.Segment(G, 49, (7, 7)),
                        W.Segment(C, 17), W.Segment(G, 100, (10, 10)), W.Segment(C, 5)],
                       rope="2d", norm=False, theta=1e4),
    "mha_g1": small([W.Segment(C, 50), W.Segment(F, 150)], hq=2, hkv=2, rope="1d"),
    "gqa_g2": small([W.Segment(C, 50), W.Segment(F, 150)], hq=4, hkv=2, rope="1d"),
    "d64": small([W.Segment(C, 45), W.Segment(G, 81, (9, 9)), W.Segment(C, 3)], d=64),
    "d64_g1": small([W.Segment(F, 70), W.Segment(C, 60)], hq=2, hkv=2, d=64, rope="none"),
    "d64_g2": small([W.Segment(C, 90), W.Segment(F, 49, (7, 7))], hq=4, hkv=2, d=64, norm=False),
    "one_token": small([W.Segment(C, 1)], batch=3),
    "all_causal": small([W.Segment(C, 300)], rope="1d"),
    "all_full": small([W.Segment(F, 200)], rope="2d", theta=1e4),
    "no_prologue": small([W.Segment(C, 37), W.Segment(F, 64, (8, 8))], rope="none", norm=False),
    "rows_before_keys_of_block": small([W.Segment(C, 3), W.Segment(F, 130)], hq=4, hkv=1),
    # Gen Images of a multi-image training sequence: hidden from every token after them
    "gen_small": small([W.Segment(C, 33), W.Segment(GEN, 64, (8, 8)), W.Segment(C, 17),
                        W.Segment(GEN, 100, (10, 10)), W.Segment(C, 5)], rope="2d", norm=False, theta=1e4),
    "gen_first": small([W.Segment(GEN, 81, (9, 9)), W.Segment(C, 100)], rope="2d", theta=1e4),
    "gen_adjacent_g2": small([W.Segment(C, 20), W.Segment(GEN, 49, (7, 7)), W.Segment(GEN, 36, (6, 6)),
                              W.Segment(G, 25, (5, 5)), W.Segment(C, 70)], hq=4, hkv=2),
    "gen_g1_d64": small([W.Segment(C, 40), W.Segment(GEN, 64, (8, 8)), W.Segment(F, 30), W.Segment(C, 60)],
                        hq=2, hkv=2, d=64),
    "gen_long": small([W.Segment(C, 130), W.Segment(GEN, 256, (16, 16)), W.Segment(C, 70),
                       W.Segment(GEN, 400, (20, 20)), W.Segment(C, 40)], rope="2d", norm=False, theta=1e4,
                      batch=1),
}


def output_grad(w, seed=77):
    rng = np.random.default_rng(seed)
    g = rng.standard_normal((w.batch, w.seq_len, w.n_q_heads, w.head_dim), dtype=np.float32)
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(g)).reshape(g.shape)


def run_train(x, dout_np):
    """Forward with lse and backward on the GPU; returns host float64 arrays."""
    w = x.workload
    dev = to_device(x)
    desc = desc_for(w, x.segments)
    pro = prologue_for(w, dev)
    ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, pro),
                         B.ha_attn_bwd_workspace_bytes(desc, pro)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    lse = torch.empty((w.batch, w.n_q_heads, w.seq_len), dtype=torch.float32, device="cuda")
    B.ha_attn_fwd_lse(desc, pro, dev["q"], dev["k"], dev["v"], out, lse, ws)
    dout = torch.from_numpy(dout_np).to(torch.bfloat16).cuda()
    dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    norm = w.qk_norm
    dwq = torch.full((w.head_dim,), float("nan"), device="cuda") if norm else None
    dwk = torch.full((w.head_dim,), float("nan"), device="cuda") if norm else None
    B.ha_attn_bwd(desc, pro, dev["q"], dev["k"], dev["v"], out, lse, dout, dq, dk, dv, dwq, dwk, ws)
    torch.cuda.synchronize()
    res = {"out": f64(out), "lse": f64(lse), "dq": f64(dq), "dk": f64(dk), "dv": f64(dv)}
    if norm:
        res["dw_q"], res["dw_k"] = f64(dwq), f64(dwk)
    return res


def check(name, got, want, bulk_gate=GRAD_ROW_BULK):
    assert np.isfinite(got).all(), f"{name}: non-finite"
    err = got - want
    rms = float(np.sqrt(np.mean(want * want)))
    mean = float(np.abs(err).mean())
    row_ref = np.sqrt(np.mean(want * want, axis=-1))
    row_err = np.sqrt(np.mean(err * err, axis=-1))
    row_rel = row_err / np.maximum(row_ref, ROW_FLOOR * rms + 1e-30)
    worst = float(row_rel.max())
    bulk = float(np.quantile(row_rel, 0.99))
    print(f"{name}: rms {rms:.3e}  row rms(err)/rms(ref): worst {worst:.3e} p99 {bulk:.3e} "
          f"median {float(np.median(row_rel)):.3e}  mean|err|/rms {mean / max(rms, 1e-30):.3e}", flush=True)
    if rms == 0.0:
        # e.g. a single token: the exact gradients are zero, and what the kernels leave is
        # fp32 residue (dP = dO.v and delta = dO.out summed in different orders), ~1e-7 per
        # term, against gradients of size ~0.1 to 10 elsewhere
        assert float(np.abs(err).max()) <= 1e-4, name
        return
    assert worst <= GRAD_ROW and bulk <= bulk_gate and mean <= GRAD_MEAN * rms, (name, worst, bulk, mean)


def check_lse(got, want):
    err = float(np.abs(got - want).max())
    print(f"lse: max|err| {err:.3e}", flush=True)
    assert err <= LSE_ABS, err


@pytest.mark.parametrize("name", sorted(SMALL))
def test_backward_small_layouts(name):
    w = SMALL[name]
    print(f"case {name}: S={w.seq_len} Hq={w.n_q_heads} Hkv={w.n_kv_heads} d={w.head_dim}", flush=True)
    x = W.generate(w)
    dout = output_grad(w)
    got = run_train(x, dout)
    masks = [oracle.explicit_mask(x.segments[b], w.seq_len) for b in range(w.batch)]
    q_rot, k_rot = oracle.prologue(x)
    check_lse(got["lse"], oracle.attention_lse(q_rot, k_rot, masks))
    want = oracle.path_backward(x, dout)
    for t in ("dq", "dk", "dv"):
        check(f"{name} {t}", got[t], want[t])
    if w.qk_norm:
        for t in ("dw_q", "dw_k"):
            check(f"{name} {t}", got[t], want[t])


@pytest.mark.parametrize("name", ["hd_small", "gca_small", "d64", "gen_small", "gen_long"])
def test_backward_two_heads_per_step(name):
    """G = 4 with dK/dV in two launches: two heads per step over 128-key blocks for the
    keys whose blocks fill two whole rounds of the CUs, four heads per step over 64-key blocks
    for the rest (gen_long: no rest). plan_cus = 2 gives these small layouts that split."""
    w = SMALL[name]
    assert w.n_q_heads // w.n_kv_heads == 4
    print(f"case {name}: S={w.seq_len} plan_cus 2", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=79)
    with plan(plan_cus=2):
        got = run_train(x, dout)
    want = oracle.path_backward(x, dout)
    for t in ("dq", "dk", "dv"):
        check(f"{name} {t}", got[t], want[t])
    if w.qk_norm:
        for t in ("dw_q", "dw_k"):
            check(f"{name} {t}", got[t], want[t])


@pytest.mark.parametrize("kind", [F, GEN])
def test_backward_tail_in_parts(kind):
    """With 4 CUs planned, 1054 keys of one KV head: keys [0, 1024) in 128-key blocks (two
    rounds of 4), the last 30 keys in one 64-key block whose 32-row steps are cut into 4
    ranges, each writing fp32 partial dK and dV that are summed in part order."""
    w = small([W.Segment(C, 30), W.Segment(kind, 1024, (32, 32))], hq=4, hkv=1, batch=1,
              rope="2d", theta=1e4)
    print(f"case tail in parts: kind {kind} S={w.seq_len} plan_cus 4", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=80)
    with plan(plan_cus=4):
        got = run_train(x, dout)
    want = oracle.path_backward(x, dout)
    for t in ("dq", "dk", "dv", "dw_q", "dw_k"):
        check(f"tail in parts {t}", got[t], want[t])


def test_backward_hd1024_full():
    """The 1024^2 HiDream layout at full size (both batch items, every head)."""
    w = W.get_config("hd1024")
    print("case hd1024: full compare", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=78)
    got = run_train(x, dout)
    want = oracle.path_backward(x, dout)
    for t in ("dq", "dk", "dv", "dw_q", "dw_k"):
        check(f"hd1024 {t}", got[t], want[t])


def test_backward_hd2048_one_group():
    """The 2048^2 layout in the benchmark's launch configuration; the oracle computes KV
    group 3 of batch item 1 (its 4 query heads' dq, its dk and dv)."""
    w = W.get_config("hd2048")
    print("case hd2048: group 3 of item 1", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=79)
    got = run_train(x, dout)
    one = dataclasses.replace(x, workload=w.replace(batch=1), q=x.q[1:], k=x.k[1:], v=x.v[1:],
                              positions=x.positions[1:], segments=x.segments[1:])
    want = oracle.path_backward(one, dout[1:], groups=[3])
    heads = slice(12, 16)
    check("hd2048 dq", got["dq"][1, :, heads], want["dq"][0, :, heads])
    check("hd2048 dk", got["dk"][1, :, 3], want["dk"][0, :, 3])
    check("hd2048 dv", got["dv"][1, :, 3], want["dv"][0, :, 3])


def test_backward_edit_one_group():
    """The editing layout at full size (text, a full 64x64 generation grid, a causal 64x64
    reference grid; S = 8448), whose dK/dV plan differs from the 2048^2 one; the oracle
    computes KV group 6 of batch item 0 (its 4 query heads' dq, its dk and dv)."""
    w = W.get_config("edit")
    print("case edit: group 6 of item 0", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=82)
    got = run_train(x, dout)
    one = dataclasses.replace(x, workload=w.replace(batch=1), q=x.q[:1], k=x.k[:1], v=x.v[:1],
                              positions=x.positions[:1], segments=x.segments[:1])
    want = oracle.path_backward(one, dout[:1], groups=[6])
    heads = slice(24, 28)
    check("edit dq", got["dq"][0, :, heads], want["dq"][0, :, heads])
    check("edit dk", got["dk"][0, :, 6], want["dk"][0, :, 6])
    check("edit dv", got["dv"][0, :, 6], want["dv"][0, :, 6])


def test_backward_multigen_one_group():
    """The multi-image training layout at full size (text, a 32x32 Gen Image, text, a
    64x64 Gen Image, text; S = 6016); the oracle computes KV group 5 (its 4 query heads'
    dq, its dk and dv)."""
    w = W.get_config("hunyuan_multigen")
    print("case hunyuan_multigen: group 5", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=80)
    got = run_train(x, dout)
    want = oracle.path_backward(x, dout, groups=[5])
    heads = slice(20, 24)
    check("multigen dq", got["dq"][0, :, heads], want["dq"][0, :, heads])
    check("multigen dk", got["dk"][0, :, 5], want["dk"][0, :, 5])
    check("multigen dv", got["dv"][0, :, 5], want["dv"][0, :, 5])


def test_backward_hunyuan_one_group():
    """The HunyuanImage interleave at full size with plain image segments (S = 6016). Its
    forward takes the split plan on 256 CUs (2 query blocks per KV head in 4 parts), so the
    lse the backward uses comes from the merge kernel; the oracle computes KV group 2."""
    w = W.get_config("hunyuan")
    print("case hunyuan: group 2", flush=True)
    x = W.generate(w)
    dout = output_grad(w, seed=81)
    got = run_train(x, dout)
    want = oracle.path_backward(x, dout, groups=[2])
    heads = slice(8, 12)
    check("hunyuan dq", got["dq"][0, :, heads], want["dq"][0, :, heads])
    check("hunyuan dk", got["dk"][0, :, 2], want["dk"][0, :, 2])
    check("hunyuan dv", got["dv"][0, :, 2], want["dv"][0, :, 2])


def test_autograd_matches_direct_calls():
    """api.hybrid_attention_train under torch autograd gives exactly what the direct calls
    give (same kernels), including the norm-weight gradients."""
    from unified_text_pixel_amd import api
    w = SMALL["edit_small"]
    x = W.generate(w)
    dev = to_device(x)
    attn = api.HybridAttention(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, "bf16",
                               x.segments, rope=w.rope, positions=dev["positions"], theta=w.rope_theta,
                               mrope_sections=w.mrope_sections, q_norm_weight=dev["w_q"],
                               k_norm_weight=dev["w_k"], eps=w.norm_eps)
    q, k, v = (dev[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    wq, wk = dev["w_q"].clone().requires_grad_(True), dev["w_k"].clone().requires_grad_(True)
    dout = torch.from_numpy(output_grad(w)).to(torch.bfloat16).cuda()
    out = api.hybrid_attention_train(attn, q, k, v, wq, wk)
    out.backward(dout)
    out2, lse = attn.forward_train(dev["q"], dev["k"], dev["v"])
    ref = attn.backward(dev["q"], dev["k"], dev["v"], out2, lse, dout)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), out2)
    for got, want in zip((q.grad, k.grad, v.grad, wq.grad, wk.grad), ref):
        assert torch.equal(got, want)


def test_backward_offsets_past_2_31_sampled():
    """Training forward and backward with q, out, dO and dq past 2^31 elements (1100 batch
    items x 2048 tokens x 8 query heads x 128; items from 1024 on lie wholly beyond element
    2^31), RMSNorm and 1D rotary: the 64-bit offsets of every backward kernel. Inputs drawn
    on the device from a seeded generator; the dq, dk, dv and lse of sampled items against
    the oracle's gradients of those items (the norm-weight gradients sum over all 1100
    items and are checked for finiteness only)."""
    from unified_text_pixel_amd import api
    nb, S, Hq, Hkv, D = 1100, 2048, 8, 2, 128
    assert 1024 * S * Hq * D == 2 ** 31
    seg = np.tile(np.array([[[0, 70, C], [70, S - 70, F]]], dtype=np.int32), (nb, 1, 1))
    w = small([W.Segment(C, 70), W.Segment(F, S - 70)], batch=nb, hq=Hq, hkv=Hkv, d=D, rope="1d")
    desc = desc_for(w, seg)
    gen = torch.Generator(device="cuda").manual_seed(17)

    def draw(h):
        t = torch.empty((nb, S, h, D), dtype=torch.bfloat16, device="cuda")
        for b0 in range(0, nb, 128):  # fp32 draws in slices, rounded to bf16
            t[b0:b0 + 128] = torch.randn((min(128, nb - b0), S, h, D), generator=gen, device="cuda")
        return t

    q, k, v, dout = draw(Hq), draw(Hkv), draw(Hkv), draw(Hq)
    wrng = np.random.default_rng(18)
    w_q = (1 + 0.02 * wrng.standard_normal(D)).astype(np.float32)
    w_k = (1 + 0.02 * wrng.standard_normal(D)).astype(np.float32)
    pos = np.broadcast_to(np.arange(S, dtype=np.int32)[None, :, None], (nb, S, 1))
    cs = api.rope_table(w.rope_theta, D, S)
    pro = B.PrologueDesc("1d", torch.from_numpy(np.ascontiguousarray(pos)).cuda(), cs, cs.shape[0],
                         torch.from_numpy(w_q).cuda(), torch.from_numpy(w_k).cuda(), w.norm_eps,
                         w.mrope_sections)
    ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, pro), B.ha_attn_bwd_workspace_bytes(desc, pro)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((nb, Hq, S), dtype=torch.float32, device="cuda")
    B.ha_attn_fwd_lse(desc, pro, q, k, v, out, lse, ws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dwq = torch.full((D,), float("nan"), device="cuda")
    dwk = torch.full((D,), float("nan"), device="cuda")
    B.ha_attn_bwd(desc, pro, q, k, v, out, lse, dout, dq, dk, dv, dwq, dwk, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dwq).all() and torch.isfinite(dwk).all()
    for b in (0, 1024, nb - 1):
        x1 = W.Inputs(workload=w.replace(batch=1), q=f64(q[b:b + 1]), k=f64(k[b:b + 1]), v=f64(v[b:b + 1]),
                      q_bits=None, k_bits=None, v_bits=None, w_q=w_q, w_k=w_k, positions=pos[b:b + 1],
                      segments=seg[b:b + 1])
        want = oracle.path_backward(x1, f64(dout[b:b + 1]))
        for name in ("dq", "dk", "dv"):
            got = f64({"dq": dq, "dk": dk, "dv": dv}[name][b:b + 1])
            check(f"item {b} of {nb} {name}", got, want[name])
        check_lse(f64(lse[b:b + 1]), oracle.path_lse(x1))


@pytest.mark.parametrize("alpha,sign", [(26.0, 1.0), (36.0, -1.0)])
def test_backward_extreme_logits(alpha, sign):
    """q and k share a strong common direction e_0, shifting every score of a row by about
    +86 or -165 log2 units (no norm, no rotary, as the HunyuanImage layouts train): the
    forward's row lse then comes from its careful re-referencing pass, and the backward's
    P = exp2(S' - log2(e) lse) must stay in range. dk, dv and dq off the common direction
    against the oracle at the usual gates. Two quantities are ill conditioned here and get
    bounds from their conditioning instead:
    - lse: both passes score with q' = bf16(scale log2(e) q), whose rounding (2^-8 relative)
      times the common component shifts a row's scores by a constant: the output does not
      see it, the lse does (as on every path that rounds q', the prologue's included); it is
      checked against ln 2 * sum_d 2^-8 |scale log2(e) q_d| max_j |k_jd| + the usual 2e-2;
    - dq along e_0, a difference of terms alpha times larger than itself (dq_i[0] = scale
      sum_j dZ_ij k_j[0] with sum_j dZ_ij = 0 exactly): its error is the rounding left in
      sum_j dZ_ij times alpha: a few bf16 roundings of dZ, and delta = rowsum(dO O) taken
      from the bf16 output. Checked against scale max|k_j[0]| (2^-7 sum_j |dZ_ij| + 2^-8
      sum_d |dO_d O_d|), dZ and O from the same inputs in float64.
    The same rounding of q' along e_0 (2^-8 |scale log2(e) q_0|, about 0.013) times each
    key's k_j[0] - mean_j k_j[0] moves every score by ~0.01 log2 units, so P and the
    gradients move by ~1%: the rows' 99th percentile is held to 2e-2 here (1e-2 on well
    conditioned inputs); the worst-row and mean gates are the usual ones."""
    w = small([W.Segment(C, 40), W.Segment(F, 100), W.Segment(G, 61)], rope="none", norm=False)
    print(f"case common direction {sign * alpha}", flush=True)
    x = W.generate(w)
    x.q[..., 0] += sign * alpha
    x.k[..., 0] += alpha
    for n in ("q", "k"):  # the inputs both sides see: rounded to bf16 again
        bits = W.f32_to_bf16_bits(getattr(x, n))
        setattr(x, n + "_bits", bits.reshape(getattr(x, n).shape))
        setattr(x, n, W.bf16_bits_to_f32(bits).reshape(getattr(x, n).shape))
    dout = output_grad(w, seed=83)
    got = run_train(x, dout)
    want = oracle.path_backward(x, dout)
    c = float(np.float32(1.0 / np.sqrt(w.head_dim) * 1.4426950408889634))
    G_ = w.n_q_heads // w.n_kv_heads
    lse_err = np.abs(got["lse"] - oracle.path_lse(x))  # [B][Hq][S]
    lse_ratio = 0.0
    for b in range(w.batch):
        for h in range(w.n_q_heads):
            kmax = np.abs(x.k[b, :, h // G_]).max(axis=0)                     # [d]
            bound = np.log(2.0) * (2.0 ** -8 * np.abs(c * x.q[b, :, h]) * kmax).sum(axis=1) + LSE_ABS
            lse_ratio = max(lse_ratio, float((lse_err[b, h] / bound).max()))
    print(f"extreme {sign * alpha} lse: max|err| {lse_err.max():.3e}, worst error / bound {lse_ratio:.3f}", flush=True)
    assert lse_ratio <= 1.0, lse_ratio
    for name in ("dk", "dv"):
        check(f"extreme {sign * alpha} {name}", got[name], want[name], bulk_gate=2e-2)
    check(f"extreme {sign * alpha} dq off e_0", got["dq"][..., 1:], want["dq"][..., 1:], bulk_gate=2e-2)
    # dq along e_0 against its conditioning bound (plus a floor of 1e-3 of the tensor's rms:
    # a row that sees one key has dZ = 0 exactly, and the kernels leave fp32 residue there)
    scale = 1.0 / np.sqrt(w.head_dim)
    floor = 1e-3 * float(np.sqrt(np.mean(want["dq"] ** 2)))
    worst = 0.0
    for b in range(w.batch):
        M = oracle.explicit_mask(x.segments[b], w.seq_len)
        for h in range(w.n_q_heads):
            g = h // G_
            q = x.q[b, :, h].astype(np.float64)
            k = x.k[b, :, g].astype(np.float64)
            v = x.v[b, :, g].astype(np.float64)
            z = np.where(M, q @ k.T * scale, -np.inf)
            pr = np.exp(z - z.max(axis=1, keepdims=True))
            pr /= pr.sum(axis=1, keepdims=True)
            do = dout[b, :, h].astype(np.float64)
            dp = do @ v.T
            dz = pr * (dp - (pr * dp).sum(axis=1, keepdims=True))
            o = pr @ v  # delta = rowsum(dO * O) is taken from O rounded to bf16 (2^-8)
            bound = scale * np.abs(k[:, 0]).max() * (2.0 ** -7 * np.abs(dz).sum(axis=1) +
                                                      2.0 ** -8 * np.abs(do * o).sum(axis=1)) + floor
            err = np.abs(got["dq"][b, :, h, 0] - want["dq"][b, :, h, 0])
            worst = max(worst, float((err / (bound + 1e-30)).max()))
    print(f"extreme {sign * alpha} dq along e_0: worst error / conditioning bound {worst:.3f}", flush=True)
    assert worst <= 1.0, worst
