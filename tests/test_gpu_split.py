"""Split query blocks in the bf16 forward (ha_attn_fwd, ha_attn_fwd_lse): the work items may
split a query block's tile list into parts, each writing an unnormalised partial output, row
sum and row reference that a merge kernel combines. The planner splits only where the heavy
blocks leave a CU round partly idle (the HunyuanImage layouts on 256 CUs); two descriptor
fields reach the other cases: split_parts = P splits every block into P parts (P = 1 never
splits) and plan_cus plans for another CU count. A kernel builds the work item table in the
workspace from the classifier's tile counts.

Each case is checked against the oracle at the usual tolerances and against the unsplit run
(same inputs; the two differ only in the fp32 summation order before the bf16 rounding)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (compare, desc_for, f64, plan, prologue_for, refresh_bits, require_gpu,
                         run_fwd, sample_rows)
from test_gpu_parity import SMALL, small
from unified_text_pixel_amd import binding as B
from workloads.device import to_device

pytestmark = pytest.mark.gpu

C, F, G, GEN = W.SEG_CAUSAL, W.SEG_FULL, W.SEG_GCA, W.SEG_GEN
LSE_ABS = 2e-2  # as for the training forward


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def fwd_lse(x, dev):
    """ha_attn_fwd_lse (ha_attn_fwd and no lse for GQA groups of 8, which the training entry
    points do not take); returns (out, lse or None, workspace bytes)."""
    w = x.workload
    desc = desc_for(w, x.segments)
    pro = prologue_for(w, dev)
    nbytes = B.ha_attn_workspace_bytes(desc, pro)
    ws = torch.empty(max(256, nbytes), dtype=torch.uint8, device="cuda")
    out = torch.full_like(dev["q"], float("nan"))
    if w.n_q_heads // w.n_kv_heads > 4:
        B.ha_attn_fwd(desc, pro, dev["q"], dev["k"], dev["v"], out, ws)
        torch.cuda.synchronize()
        return out, None, nbytes
    lse = torch.full((w.batch, w.n_q_heads, w.seq_len), float("nan"), dtype=torch.float32,
                     device="cuda")
    B.ha_attn_fwd_lse(desc, pro, dev["q"], dev["k"], dev["v"], out, lse, ws)
    torch.cuda.synchronize()
    return out, lse, nbytes


def close_to_unsplit(got, ref, what):
    """Same inputs, another fp32 summation order: at most a couple of bf16 ulps apart."""
    a, b = f64(got), f64(ref)
    tol = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -14
    bad = np.abs(a - b) > tol
    print(f"{what}: max|split - unsplit| {np.abs(a - b).max():.3e}", flush=True)
    assert not bad.any(), (what, int(bad.sum()))


FORCED = ["hd_small", "edit_small", "gca_small", "gqa_g8", "mha_g1", "d64_bf16", "one_token",
          "causal_rows_in_long_block", "all_full", "gen_small", "gen_first", "gen_adjacent",
          "gen_g1_d64"]


@pytest.mark.parametrize("parts", [2, 5])
@pytest.mark.parametrize("name", FORCED)
def test_forced_split_small(name, parts):
    """Every block in 2 or 5 parts: parts of one tile, empty parts (5 parts of blocks with
    fewer tiles), masked tiles in any part, Gen Image holes; output and lse against the
    oracle and against the unsplit run."""
    w = SMALL[name]
    print(f"case {name}: parts {parts} S={w.seq_len}", flush=True)
    x = W.generate(w)
    dev = to_device(x)
    with plan(split_parts=1):
        ref, ref_lse, n0 = fwd_lse(x, dev)
    with plan(split_parts=parts):
        out, lse, n1 = fwd_lse(x, dev)
        plain, _ = run_fwd(x, dev)
    assert n1 > n0, "the split plan was not taken"
    compare(f64(out), oracle.hot_path(x), "bf16", f"{name} in {parts} parts")
    close_to_unsplit(out, ref, name)
    assert torch.equal(plain, out), "ha_attn_fwd and ha_attn_fwd_lse differ on the split path"
    if lse is not None:
        err = float(np.abs(f64(lse) - oracle.path_lse(x)).max())
        print(f"{name}: lse max|err| {err:.3e}", flush=True)
        assert err <= LSE_ABS, err
        assert float((lse - ref_lse).abs().max()) <= 1e-4


@pytest.mark.parametrize("name", ["hd_small", "gen_small", "one_token"])
def test_forced_split_most_parts(name):
    """64 parts, the most split_parts takes: every block has at most 6 key tiles here, so
    most parts are empty and each block's merge sees parts of one tile between them."""
    w = SMALL[name]
    x = W.generate(w)
    dev = to_device(x)
    with plan(split_parts=1):
        ref, _, n0 = fwd_lse(x, dev)
    with plan(split_parts=64):
        out, lse, n1 = fwd_lse(x, dev)
    assert n1 > n0
    compare(f64(out), oracle.hot_path(x), "bf16", f"{name} in 64 parts")
    close_to_unsplit(out, ref, name)
    assert float(np.abs(f64(lse) - oracle.path_lse(x)).max()) <= LSE_ABS


@pytest.mark.parametrize("alpha,sign", [(26.0, 1.0), (36.0, -1.0)])
def test_forced_split_careful_pass(alpha, sign):
    """Scores shifted by +86 or -165 log2 units: the parts take the careful re-referencing
    pass, so the merge combines partial results on different references."""
    w = small([W.Segment(C, 40), W.Segment(F, 100), W.Segment(G, 61)], rope="none", norm=False,
              hq=8, hkv=2)
    x = W.generate(w)
    x.q[..., 0] += sign * alpha
    x.k[..., 0] += alpha
    refresh_bits(x)
    dev = to_device(x)
    with plan(split_parts=3):
        out, _ = run_fwd(x, dev)
    compare(f64(out), oracle.hot_path(x), "bf16", f"split, extreme logits {sign * alpha}")


def test_forced_split_late_keys_one_head():
    """Only head 3 and keys from 130 on carry the shift: in a split block some parts take the
    careful pass and others do not."""
    w = small([W.Segment(C, 40), W.Segment(F, 100), W.Segment(G, 61)], rope="none", norm=False,
              hq=8, hkv=2)
    x = W.generate(w)
    x.q[:, :, 3, 0] += 26.0
    x.k[:, 130:, :, 0] += 26.0
    refresh_bits(x)
    dev = to_device(x)
    with plan(split_parts=2):
        out, _ = run_fwd(x, dev)
    compare(f64(out), oracle.hot_path(x), "bf16", "split, late extreme keys in one head")


@pytest.mark.parametrize("name,cus", [("hunyuan", None), ("hunyuan_multigen", 240),
                                      ("hunyuan", 240), ("hd2048", 240), ("hd2048", 304)])
def test_planner_full_size(name, cus):
    """The planner on full-size layouts, for this device's CU count (None) or another one:
    sampled rows against the oracle, every output and lse against the unsplit run."""
    w = W.get_config(name)
    print(f"case {name}: cus {cus}", flush=True)
    x = W.generate(w)
    dev = to_device(x)
    with plan(split_parts=1):
        ref, ref_lse, n0 = fwd_lse(x, dev)
    with plan(plan_cus=cus or 0):
        out, lse, n1 = fwd_lse(x, dev)
    if cus is None and n1 == n0:
        pytest.skip("this device's CU count gives no split for this layout")
    assert n1 > n0, "the split plan was not taken"
    got = f64(out)
    rows = sample_rows(w)
    for b in range(w.batch):
        want = oracle.hot_path_rows(x, b, rows, list(range(w.n_q_heads)))
        compare(got[b, rows], want, w.dtype, f"{name} batch {b}, split")
    close_to_unsplit(out, ref, name)
    assert float((lse - ref_lse).abs().max()) <= 1e-4


def test_split_with_short_workspace_runs_unsplit():
    """A workspace sized for the unsplit path (smaller than ha_attn_workspace_bytes asks for
    with a split plan) runs unsplit rather than failing."""
    w = SMALL["gca_small"]
    x = W.generate(w)
    dev = to_device(x)
    pro = prologue_for(w, dev)
    with plan(split_parts=1):
        n0 = B.ha_attn_workspace_bytes(desc_for(w, x.segments), pro)
        ref, _ = run_fwd(x, dev)
    with plan(split_parts=4):
        desc = desc_for(w, x.segments)
    assert B.ha_attn_workspace_bytes(desc, pro) > n0
    ws = torch.empty(n0, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    B.ha_attn_fwd(desc, pro, dev["q"], dev["k"], dev["v"], out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_planner_pads_per_batch_lists():
    """Two batch items with different layouts on 4 KV heads: XCDs 0-3 serve item 0 and 4-7
    item 1, their sorted lists differ, so the table pads the shorter ones with empty entries.
    For 96 CUs: 176 entries, 24 of them padding, 12 split blocks (see the split planner's
    host tests for the sizes). Output and lse against the oracle and the unsplit run."""
    w = small([W.Segment(C, 100), W.Segment(F, 900, (30, 30))], hq=16, hkv=4, batch=2)
    x = W.generate(w)
    seg = W.segment_table(w)
    seg[1] = [[0, 700, C], [700, 300, G]]
    x.segments = seg
    dev = to_device(x)
    with plan(split_parts=1):
        ref, ref_lse, n0 = fwd_lse(x, dev)
    with plan(plan_cus=96):
        out, lse, n1 = fwd_lse(x, dev)
    assert n1 > n0, "the split plan was not taken"
    compare(f64(out), oracle.hot_path(x), "bf16", "per-batch layouts, padded item table")
    close_to_unsplit(out, ref, "per-batch layouts")
    err = float(np.abs(f64(lse) - oracle.path_lse(x)).max())
    assert err <= LSE_ABS, err
    assert float((lse - ref_lse).abs().max()) <= 1e-4


def _r256(n):
    return (n + 255) // 256 * 256


def _block_costs(w, segments, bq):
    """Key tiles each (batch item, query block) executes: the non-SKIP tiles of the oracle's
    brute-force labels over the explicit mask (query blocks aligned to the sequence end)."""
    out = []
    for b in range(w.batch):
        M = oracle.explicit_mask(segments[b], w.seq_len)
        lab = oracle.tile_labels(M, bq, 64, q_end_aligned=True)
        out.append((lab != 0).sum(axis=1))
    return np.array(out)


@pytest.mark.parametrize("case", ["hunyuan_256", "per_batch_96", "forced_3", "forced_gen_2"])
def test_device_table_is_a_sorted_cover(case):
    """The work item table the plan kernel writes into the workspace: every (batch, KV head,
    query block) once, whole or as parts 0..P-1 on consecutive slots with a matching split
    row; each entry on the XCD of its pair (when the pairs split evenly over 8); each XCD's
    list longest first by key tiles (a part counts ceil(tiles / P)), padding only at the end."""
    if case == "hunyuan_256":
        w, segs, kw, sizes = W.get_config("hunyuan"), None, dict(plan_cus=256), (800, 16, 64)
    elif case == "per_batch_96":
        w = small([W.Segment(C, 100), W.Segment(F, 900, (30, 30))], hq=16, hkv=4, batch=2)
        segs = W.segment_table(w)
        segs[1] = [[0, 700, C], [700, 300, G]]
        kw, sizes = dict(plan_cus=96), (176, 12, 36)
    elif case == "forced_3":
        w, segs, kw, sizes = SMALL["hd_small"], None, dict(split_parts=3), None
    else:
        w, segs, kw, sizes = SMALL["gen_small"], None, dict(split_parts=2), None
    x = W.generate(w)
    if segs is not None:
        x.segments = segs
    segs = x.segments
    dev = to_device(x)
    with plan(**kw):
        desc = desc_for(w, segs)
    pro = prologue_for(w, dev)
    bq, _, nq, _ = B.ha_tile_shape(desc)
    grp = w.n_q_heads // w.n_kv_heads
    nbg = w.batch * w.n_kv_heads
    if sizes is None:
        P = kw["split_parts"]
        sizes = (P * nbg * nq, nbg * nq, P * nbg * nq)
    n_items, n_splits, n_slots = sizes
    total = B.ha_attn_workspace_bytes(desc, pro)
    per = n_slots * bq * grp
    plan_bytes = _r256((n_items + n_splits) * 16) + _r256(per * w.head_dim * 4) + 2 * _r256(per * 4)
    ws = torch.full((total,), 0x7F, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    B.ha_attn_fwd(desc, pro, dev["q"], dev["k"], dev["v"], out, ws)
    torch.cuda.synchronize()
    off = total - plan_bytes
    tab = ws[off:off + (n_items + n_splits) * 16].cpu().numpy().view(np.int32).reshape(-1, 4)
    items, splits = tab[:n_items], tab[n_items:]
    cost = _block_costs(w, segs, bq)
    groups = 8 if nbg % 8 == 0 else 1
    seen = {}
    split_rows = {(int(r[0]), int(r[1])): (int(r[2]), int(r[3])) for r in splits}
    assert len(split_rows) == n_splits
    for x_ in range(groups):
        lst = items[x_::groups]
        valid = lst[:, 0] >= 0
        nv = int(valid.sum())
        assert valid[:nv].all() and not valid[nv:].any(), f"padding inside the list of group {x_}"
        prev = None
        for e in lst[:nv]:
            bg, qb, pp, slot = (int(v) for v in e)
            part, parts = pp & 0xFFFF, pp >> 16
            if groups == 8:
                assert bg % 8 == x_
            c = int(cost[bg // w.n_kv_heads, qb])
            c = -(-c // parts)
            assert prev is None or c <= prev, f"group {x_} not longest first"
            prev = c
            seen.setdefault((bg, qb), []).append((part, parts, slot))
    assert set(seen) == {(bg, qb) for bg in range(nbg) for qb in range(nq)}
    used = []
    for key, ent in seen.items():
        parts = ent[0][1]
        if parts == 1:
            assert ent == [(0, 1, -1)], (key, ent)
            assert key not in split_rows
        else:
            assert sorted(p for p, _, _ in ent) == list(range(parts)) and all(e[1] == parts for e in ent)
            s0 = min(s for _, _, s in ent)
            assert sorted(s for _, _, s in ent) == list(range(s0, s0 + parts))
            assert split_rows[key] == (s0, parts)
            used.extend(range(s0, s0 + parts))
    assert sorted(used) == list(range(n_slots))
    compare(f64(out) if w.seq_len < 2000 else f64(out)[0, sample_rows(w)],
            oracle.hot_path(x) if w.seq_len < 2000 else
            oracle.hot_path_rows(x, 0, sample_rows(w), list(range(w.n_q_heads))), "bf16", case)
