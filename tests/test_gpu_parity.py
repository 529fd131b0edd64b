"""HIP path against the oracle, through the C ABI, on seeded inputs.

Small cases compare every output element; the five full-size workloads compare sampled
rows (all heads) that the oracle computes one by one, in the launch configuration the
benchmark times, plus properties that hold at any size."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (compare, desc_for, f64, plan, prologue_for, refresh_bits, require_gpu,
                         run_fwd, sample_rows, unsplit)
from unified_text_pixel_amd import api, binding as B
from workloads.device import to_device

pytestmark = pytest.mark.gpu

C, F, G, GEN = W.SEG_CAUSAL, W.SEG_FULL, W.SEG_GCA, W.SEG_GEN


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def small(segs, hq=8, hkv=2, d=128, rope="mrope", sections=None, norm=True, batch=2,
          dtype="bf16", theta=5e6, seed=21):
    if sections is None:
        sections = (24, 20, 20) if d == 128 else (12, 10, 10)
    return W.Workload(name="small", description="", batch=batch, segments=tuple(segs),
                      n_q_heads=hq, n_kv_heads=hkv, head_dim=d, dtype=dtype, rope=rope,
                      rope_theta=theta, mrope_sections=sections, qk_norm=norm, norm_eps=1e-6,
                      seed=seed)


SMALL = {
    # HiDream-style: causal prefix (ragged vs the 64-key tile) then a full grid
    "hd_small": small([W.Segment(C, 70), W.Segment(F, 256, (16, 16))]),
    # editing layout: text, full generation, causal reference; S not a tile multiple
    "edit_small": small([W.Segment(C, 40), W.Segment(F, 100, (10, 10)), W.Segment(C, 81, (9, 9))]),
    # HunyuanImage-style interleave with adjacent image segments, 2D rotary, no q/k norm
    "gca_small": small([W.Segment(C, 33), W.Segment(G, 64, (8, 8)), W.Segment(G, 49, (7, 7)),
                        W.Segment(C, 17), W.Segment(G, 100, (10, 10)), W.Segment(C, 5)],
                       rope="2d", norm=False, theta=1e4),
    "mha_g1": small([W.Segment(C, 50), W.Segment(F, 150)], hq=2, hkv=2, rope="1d"),
    "gqa_g2": small([W.Segment(C, 50), W.Segment(F, 150)], hq=4, hkv=2, rope="1d"),
    "gqa_g8": small([W.Segment(F, 90), W.Segment(C, 111)], hq=16, hkv=2, rope="none", norm=True),
    "d64_bf16": small([W.Segment(C, 45), W.Segment(G, 81, (9, 9)), W.Segment(C, 3)], d=64,
                      rope="mrope"),
    "one_token": small([W.Segment(C, 1)], batch=3),
    # rows 0-2 see keys of one lane half only, in a query block that spans several key
    # tiles (the full rows after them): the row state must stay whole across lane pairs
    "causal_rows_in_long_block": small([W.Segment(C, 3), W.Segment(F, 130)], hq=4, hkv=1),
    "all_causal": small([W.Segment(C, 300)], rope="1d"),
    "all_full": small([W.Segment(F, 200)], rope="2d", theta=1e4),
    "f32_mixed": small([W.Segment(C, 20), W.Segment(F, 36, (6, 6)), W.Segment(G, 25, (5, 5))],
                       dtype="f32", hq=4, hkv=1, d=64, rope="2d", theta=1e4),
    "f32_d128": small([W.Segment(C, 30), W.Segment(F, 70)], dtype="f32", hq=8, hkv=2, d=128,
                      rope="mrope"),
    # Gen Images (multi-image training): each hidden from every token after it
    "gen_small": small([W.Segment(C, 33), W.Segment(GEN, 64, (8, 8)), W.Segment(C, 17),
                        W.Segment(GEN, 100, (10, 10)), W.Segment(C, 5)], rope="2d", norm=False,
                       theta=1e4),
    "gen_adjacent": small([W.Segment(C, 20), W.Segment(GEN, 49, (7, 7)), W.Segment(GEN, 36, (6, 6)),
                           W.Segment(G, 25, (5, 5)), W.Segment(C, 70)]),
    # the first key tiles hidden from every later row (rows whose first listed tiles are empty)
    "gen_first": small([W.Segment(GEN, 81, (9, 9)), W.Segment(C, 100)], rope="2d", theta=1e4),
    "gen_then_full": small([W.Segment(C, 10), W.Segment(GEN, 64, (8, 8)), W.Segment(F, 64, (8, 8)),
                            W.Segment(C, 30)]),
    "gen_g8": small([W.Segment(C, 40), W.Segment(GEN, 64, (8, 8)), W.Segment(C, 100)], hq=16, hkv=2,
                    rope="none"),
    "gen_g1_d64": small([W.Segment(C, 40), W.Segment(GEN, 64, (8, 8)), W.Segment(C, 60)], hq=2, hkv=2,
                        d=64),
    "f32_gen": small([W.Segment(C, 20), W.Segment(GEN, 36, (6, 6)), W.Segment(C, 25)], dtype="f32",
                     hq=4, hkv=1, d=64, rope="2d", theta=1e4),
}


# ---------------------------------------------------------------- classifier
def classify(w, segments=None):
    desc = desc_for(w, segments)
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    labels = torch.empty((w.batch, nq, nk), dtype=torch.uint8, device="cuda")
    ranges = torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda")
    lim = torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")
    B.ha_classify_tiles(desc, labels, ranges, lim)
    torch.cuda.synchronize()
    return (bq, bk), labels.cpu().numpy(), ranges.cpu().numpy(), lim.cpu().numpy()


def check_labels(w, segments):
    """Labels against the oracle's brute force over the mask (Gen Image holes included);
    row limits and ranges describe the key prefixes before any hole, i.e. those of the same
    layout with every Gen Image as a plain image segment."""
    (bq, bk), labels, ranges, lim = classify(w, segments)
    for b in range(w.batch):
        M = oracle.explicit_mask(segments[b], w.seq_len)
        want = oracle.tile_labels(M, bq, bk, q_end_aligned=True)
        assert np.array_equal(labels[b], want), f"batch {b}: tile labels differ"
        pre = np.array(segments[b])
        pre[pre[:, 2] == GEN, 2] = G
        Mp = oracle.explicit_mask(pre, w.seq_len)
        assert np.array_equal(lim[b], Mp.sum(axis=1)), f"batch {b}: row limits differ"
        wp = oracle.tile_labels(Mp, bq, bk, q_end_aligned=True)
        kfull = (wp == 1).sum(axis=1)
        kend = wp.shape[1] - (wp == 0).sum(axis=1)
        assert np.array_equal(ranges[b, :, 0], kfull) and np.array_equal(ranges[b, :, 1], kend)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_classifier_bit_exact_configs(name):
    w = W.get_config(name)
    check_labels(w, W.segment_table(w))


def test_classifier_bit_exact_random_layouts():
    rng = np.random.default_rng(5)
    for trial in range(25):
        n = int(rng.integers(1, 9))
        batch = int(rng.integers(1, 4))
        S = int(rng.integers(n, 700))
        tables = []
        for b in range(batch):
            cuts = np.sort(rng.choice(np.arange(1, S), size=n - 1, replace=False)) if n > 1 else []
            bounds = [0, *cuts, S]
            kinds = rng.integers(0, 4, size=n)  # Gen Images included
            tables.append([[bounds[s], bounds[s + 1] - bounds[s], kinds[s]] for s in range(n)])
        seg = np.array(tables, dtype=np.int32)
        w = small([W.Segment(C, S)], batch=batch, hq=[8, 4, 16, 2][trial % 4], hkv=2)
        check_labels(w, seg)


def test_classifier_many_batch_items():
    # more segment rows than one launch's kernel arguments hold: several launches
    w = small([W.Segment(C, 10), W.Segment(G, 30), W.Segment(F, 25)], batch=50)
    seg = W.segment_table(w)
    seg[1::3, 1:, 2] = [F, G]
    check_labels(w, seg)


def test_classifier_max_sequence_sampled():
    """The largest sequence the descriptor admits (HA_MAX_SEQ_LEN = 2^22 tokens), two batch
    items with every prefix kind and cuts that are not tile multiples: the row limits of
    sampled rows (segment edges, both ends, random rows) and the ranges of the query blocks
    holding segment edges against the oracle's mask rows, ranges through the tile-label
    definition (any / all over each tile of the block). The whole mask, 2^44 pairs, is out
    of reach."""
    S = 1 << 22  # HA_MAX_SEQ_LEN of include/ha_attn.h
    seg = np.array([
        [[0, 1000, C], [1000, 2_000_000, F], [2_001_000, 1_048_576, G], [3_049_576, 777, C],
         [3_050_353, S - 3_050_353, G]],
        [[0, 333, C], [333, 1_000_003, G], [1_000_336, 65_536, G], [1_065_872, 3_000_000, F],
         [4_065_872, S - 4_065_872, C]],
    ], dtype=np.int32)
    w = small([W.Segment(C, S)], batch=2, hq=4, hkv=1)  # the descriptor's shape only
    desc = desc_for(w, seg)
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    ranges = torch.empty((2, nq, 2), dtype=torch.int32, device="cuda")
    lim = torch.empty((2, S), dtype=torch.int32, device="cuda")
    B.ha_classify_tiles(desc, None, ranges, lim)
    torch.cuda.synchronize()
    ranges, lim = ranges.cpu().numpy(), lim.cpu().numpy()
    rng = np.random.default_rng(7)
    q0 = S - nq * bq
    for b in range(2):
        edges = {e for s0, L, _ in seg[b] for e in (s0, s0 + 1, s0 + L - 1, s0 + L - 2)} | {0, S - 1}
        rows = np.array(sorted({r for r in edges if 0 <= r < S} | set(rng.integers(0, S, 16).tolist())))
        M = oracle.mask_rows(seg[b], S, rows)
        n = M.sum(axis=1)
        assert all(M[r, :n[r]].all() for r in range(len(rows))), "oracle rows are not prefixes"
        assert np.array_equal(lim[b, rows], n), f"batch {b}: row limits differ"
        for qb in sorted({(int(s0) - q0) // bq for s0, _, _ in seg[b]} | {nq - 1}):
            r0, r1 = max(q0 + qb * bq, 0), q0 + (qb + 1) * bq
            Mb = oracle.mask_rows(seg[b], S, np.arange(r0, r1)).reshape(r1 - r0, nk, bk)
            full, none = Mb.all(axis=(0, 2)), ~Mb.any(axis=(0, 2))
            want = (int(full.sum()), int(nk - none.sum()))
            assert tuple(ranges[b, qb]) == want, f"batch {b} block {qb}: ranges {tuple(ranges[b, qb])} != {want}"


def test_offsets_past_2_31_sampled():
    """q and out past 2^31 elements (1100 batch items x 2048 tokens x 8 query heads x 128;
    items from 1024 on lie wholly beyond element 2^31): the 64-bit offsets of the
    classifier, the q/k prologue (RMSNorm, 1D rotary), the attention kernel and its stores.
    Inputs drawn on the device from a seeded generator; sampled items, rows and every head
    against the oracle's whole path on those items' tensors."""
    nb, S, Hq, Hkv, D = 1100, 2048, 8, 2, 128
    assert 1024 * S * Hq * D == 2 ** 31
    seg = np.tile(np.array([[[0, 70, C], [70, S - 70, F]]], dtype=np.int32), (nb, 1, 1))
    w = small([W.Segment(C, 70), W.Segment(F, S - 70)], batch=nb, hq=Hq, hkv=Hkv, d=D, rope="1d")
    desc = desc_for(w, seg)
    gen = torch.Generator(device="cuda").manual_seed(13)

    def draw(h):
        t = torch.empty((nb, S, h, D), dtype=torch.bfloat16, device="cuda")
        for b0 in range(0, nb, 128):  # fp32 draws in slices, rounded to bf16
            t[b0:b0 + 128] = torch.randn((min(128, nb - b0), S, h, D), generator=gen, device="cuda")
        return t

    q, k, v = draw(Hq), draw(Hkv), draw(Hkv)
    wrng = np.random.default_rng(14)
    w_q = (1 + 0.02 * wrng.standard_normal(D)).astype(np.float32)
    w_k = (1 + 0.02 * wrng.standard_normal(D)).astype(np.float32)
    pos = np.broadcast_to(np.arange(S, dtype=np.int32)[None, :, None], (nb, S, 1))
    dev_pos = torch.from_numpy(np.ascontiguousarray(pos)).cuda()
    cs = api.rope_table(w.rope_theta, D, S)
    pro = B.PrologueDesc("1d", dev_pos, cs, cs.shape[0], torch.from_numpy(w_q).cuda(),
                         torch.from_numpy(w_k).cuda(), w.norm_eps, w.mrope_sections)
    out = torch.empty_like(q)
    ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, pro)), dtype=torch.uint8, device="cuda")
    B.ha_attn_fwd(desc, pro, q, k, v, out, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.array(sorted({0, 1, 69, 70, 71, 1000, S - 1} | set(rng.integers(0, S, 8).tolist())))
    heads = list(range(Hq))
    for b in (0, 1023, 1024, nb - 1):
        x1 = W.Inputs(workload=w.replace(batch=1), q=f64(q[b:b + 1]), k=f64(k[b:b + 1]), v=f64(v[b:b + 1]),
                      q_bits=None, k_bits=None, v_bits=None, w_q=w_q, w_k=w_k, positions=pos[b:b + 1],
                      segments=seg[b:b + 1])
        want = oracle.hot_path_rows(x1, 0, rows, heads)
        compare(f64(out[b, rows]), want, "bf16", f"item {b} of {nb} ({len(rows)} rows x {Hq} heads)")


# ---------------------------------------------------------------- prologue
@pytest.mark.parametrize("name", ["hd_small", "gca_small", "d64_bf16", "f32_mixed", "f32_d128"])
def test_prologue_parity(name):
    w = SMALL[name]
    x = W.generate(w)
    dev = to_device(x)
    desc, pro = desc_for(w), prologue_for(w, dev)
    qo, ko = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
    B.ha_qk_prologue(desc, pro, dev["q"], dev["k"], qo, ko)
    torch.cuda.synchronize()
    q_ref, k_ref = oracle.prologue(x)
    for got, want in ((f64(qo), q_ref), (f64(ko), k_ref)):
        if w.dtype == "bf16":  # one bf16 rounding of an fp32 result: within 1 ulp (2^-7 relative)
            assert (np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-6).all()
        else:
            assert np.abs(got - want).max() <= 1e-5 * np.abs(want).max()


@pytest.mark.parametrize("name", ["hd1024", "hunyuan"])
def test_prologue_parity_full_size_in_place(name):
    w = W.get_config(name)
    x = W.generate(w)
    dev = to_device(x)
    desc, pro = desc_for(w), prologue_for(w, dev)
    B.ha_qk_prologue(desc, pro, dev["q"], dev["k"], dev["q"], dev["k"])  # aliasing allowed
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = rng.integers(0, w.seq_len, size=64)
    sub = W.Inputs(workload=w.replace(batch=1), q=x.q[:1, rows], k=x.k[:1, rows], v=x.v[:1, rows],
                   q_bits=None, k_bits=None, v_bits=None, w_q=x.w_q, w_k=x.w_k,
                   positions=x.positions[:1, rows], segments=x.segments[:1])
    q_ref, k_ref = oracle.prologue(sub)
    for got, want in ((f64(dev["q"][0, rows]), q_ref[0]), (f64(dev["k"][0, rows]), k_ref[0])):
        assert (np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-6).all()


# ---------------------------------------------------------------- attention
@pytest.mark.parametrize("name", list(SMALL))
def test_attention_parity_small(name):
    w = SMALL[name]
    x = W.generate(w)
    out, _ = run_fwd(x)
    compare(f64(out), oracle.hot_path(x), w.dtype, name)


def test_tiny_config_fp32():
    w = W.get_config("tiny")
    x = W.generate(w)
    out, _ = run_fwd(x)
    compare(f64(out), oracle.hot_path(x), "f32", "tiny")


@pytest.mark.parametrize("name", ["hd1024", "hd2048", "edit", "hunyuan", "hunyuan_multigen"])
def test_full_size_sampled_rows(name):
    w = W.get_config(name)
    x = W.generate(w)
    out, dev = run_fwd(x)
    got = f64(out)
    rows = sample_rows(w)
    heads = list(range(w.n_q_heads))
    errs = []
    for b in range(w.batch):
        want = oracle.hot_path_rows(x, b, rows, heads)
        errs.append(np.abs(got[b, rows] - want))
        compare(got[b, rows], want, w.dtype, f"{name} batch {b} ({len(rows)} rows x {len(heads)} heads)")
    # row 0 is causal text: it attends only to itself, so its output is v_0 exactly
    v0 = f64(dev["v"][:, 0])
    assert np.array_equal(got[:, 0], np.repeat(v0, w.n_q_heads // w.n_kv_heads, axis=1))


@pytest.mark.parametrize("name,group", [("hd2048", 3), ("edit", 6), ("hunyuan", 1), ("hunyuan_multigen", 5)])
def test_full_size_kv_group_whole(name, group):
    """Every row of every batch item for the G query heads of one KV head, at the full size
    of the workload and in the launch configuration ha_attn_fwd chooses (the split plan on
    the HunyuanImage layout, tile lists with Gen Images)."""
    w = W.get_config(name)
    x = W.generate(w)
    out, _ = run_fwd(x)
    G = w.n_q_heads // w.n_kv_heads
    heads = list(range(group * G, (group + 1) * G))
    want = oracle.hot_path(x, heads=heads)[:, :, heads]
    compare(f64(out)[:, :, heads], want, w.dtype, f"{name} KV group {group}, whole ({w.seq_len} rows x {G} heads)")


SLICE_CASES = {
    "page1024": W.page_shape_configs()["page1024"],
    "hd_small": SMALL["hd_small"],
    "edit_small": SMALL["edit_small"],
    "gca_small": SMALL["gca_small"],
    "d64_bf16": SMALL["d64_bf16"],
    "causal_rows_in_long_block": SMALL["causal_rows_in_long_block"],
}


@pytest.mark.parametrize("name", list(SLICE_CASES))
def test_slice_workgroups_match_whole_blocks(name):
    """With fewer work items than CUs (GQA group 4, plain tile ranges) every 32-row slice of a
    query block runs as a workgroup of its own. Each row computes exactly as in a workgroup
    that covers the whole block, so the two launches (the second planned for one CU, where
    the items are not fewer than the CUs) agree bit for bit, output and row lse, and both
    match the oracle."""
    w = SLICE_CASES[name]
    x = W.generate(w)
    dev = to_device(x)
    pro = prologue_for(w, dev)
    res = []
    for cus in (0, 1):
        with plan(split_parts=1, plan_cus=cus):
            desc = desc_for(w, x.segments)
        ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, pro)), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(dev["q"])
        lse = torch.empty((w.batch, w.n_q_heads, w.seq_len), dtype=torch.float32, device="cuda")
        B.ha_attn_fwd_lse(desc, pro, dev["q"], dev["k"], dev["v"], out, lse, ws)
        torch.cuda.synchronize()
        res.append((out, lse))
    assert torch.equal(res[0][0], res[1][0]), "output differs between slice and whole-block workgroups"
    assert torch.equal(res[0][1], res[1][1]), "row lse differs between slice and whole-block workgroups"
    compare(f64(res[0][0]), oracle.hot_path(x), w.dtype, f"{name} in slice workgroups")


def test_hd1024_whole_output():
    """The 1024^2 HiDream-style workload (batch 2, 1282 tokens, 32 heads) compared with the
    oracle on every output element, in the launch configuration ha_attn_fwd chooses."""
    w = W.get_config("hd1024")
    x = W.generate(w)
    out, _ = run_fwd(x)
    compare(f64(out), oracle.hot_path(x), w.dtype, "hd1024 whole output")


def test_long_sequence_sampled_rows():
    """A 4096^2 HiDream-style image: 258 causal tokens then a 128 x 128 grid of full rows
    (S = 16642, 261 key tiles per generation row), batch 1, sampled rows against the
    oracle; large grids, long key loops and wide indices."""
    w = W.get_config("hd2048").replace(
        name="hd4096", batch=1,
        segments=(W.Segment(C, 258), W.Segment(F, 128 * 128, (128, 128))))
    x = W.generate(w)
    out, _ = run_fwd(x)
    got = f64(out)
    rows = sample_rows(w, n_random=24)
    heads = list(range(0, w.n_q_heads, 3))
    want = oracle.hot_path_rows(x, 0, rows, heads)
    compare(got[0, rows][:, heads], want, w.dtype, f"hd4096 ({len(rows)} rows x {len(heads)} heads)")


@pytest.mark.parametrize("kinds", [[C, F, G], [C, F, G, GEN]], ids=["plain", "gen"])
def test_max_segment_count(kinds):
    """64 segments per item (the most a table may hold), random kinds and lengths, image
    segments side by side, two items with different tables: whole output against the
    oracle."""
    rng = np.random.default_rng(11)
    S = 700
    segs = []
    for b in range(2):
        lens = rng.integers(1, 11, size=64)
        lens[-1] += S - lens.sum()
        at, rows = 0, []
        for L, k in zip(lens, rng.integers(0, len(kinds), size=64)):
            rows.append([at, int(L), kinds[int(k)]])
            at += int(L)
        segs.append(rows)
    seg = np.array(segs, dtype=np.int32)
    w = small([W.Segment(C, S)], batch=2, rope="1d")
    x = W.generate(w)
    x.segments = seg
    check_labels(w, seg)
    out, _ = run_fwd(x)
    compare(f64(out), oracle.hot_path(x), "bf16", "64 segments")


def test_careful_pass_full_size_shape():
    """The hd1024 layout at full size with every score of query head 5 shifted by about +86
    log2 units from key 300 on: the work items of that head's KV group take the careful
    pass across all of their tiles; sampled rows against the oracle. Without a rotary
    embedding the shift is the same for every key of a row, so the bf16 rounding of the
    large prescaled q component cancels in the softmax (with rotation it would not, and the
    comparison would measure bf16 conditioning instead of the careful pass)."""
    w = W.get_config("hd1024").replace(qk_norm=False, batch=1, rope="none")
    x = W.generate(w)
    x.q[:, :, 5, 0] += 26.0
    x.k[:, 300:, :, 0] += 26.0
    out, _ = run_fwd(refresh_bits(x))
    got = f64(out)
    rows = sample_rows(w, n_random=16)
    heads = [4, 5, 6, 7, 12]
    want = oracle.hot_path_rows(x, 0, rows, heads)
    compare(got[0, rows][:, heads], want, w.dtype, f"careful pass at hd1024 shape")


def uniform_probe(w):
    """q = 0 makes every allowed weight exactly 1 (RMSNorm and rotary of 0 are 0), masked
    ones exactly 0; with v_j one-hot on channel (j // 64) mod d the output channel c of row
    i is the count of allowed keys in the 64-key blocks on c, over the row's allowed keys."""
    x = W.generate(w)
    x.q[:] = 0.0
    S, d = w.seq_len, w.head_dim
    x.v[:] = 0.0
    chan = (np.arange(S) // 64) % d
    x.v[:, np.arange(S), :, chan] = 1.0
    out, _ = run_fwd(refresh_bits(x))
    got = f64(out)
    for b in range(w.batch):
        M = oracle.explicit_mask(x.segments[b], S)
        for i in np.unique(np.r_[np.arange(0, S, 7), S - 1]):
            keys = np.nonzero(M[i])[0]
            want = np.bincount(chan[keys], minlength=d) / len(keys)
            tol = 2.0 ** -7 * want + 1e-7
            assert (np.abs(got[b, i] - want[None, :]) <= tol).all(), (w.name, b, i)


@pytest.mark.parametrize("name", ["hd2048", "edit", "hunyuan", "hunyuan_multigen"])
def test_uniform_probe_full_size(name):
    uniform_probe(W.get_config(name))


@pytest.mark.parametrize("name", ["hd_small", "edit_small", "gca_small", "all_full", "gen_small",
                                  "gen_first", "f32_gen"])
def test_uniform_probe_small(name):
    uniform_probe(SMALL[name])


def test_future_tokens_do_not_leak():
    w = SMALL["gca_small"].replace(batch=1)
    x = W.generate(w)
    base, _ = run_fwd(x)
    # segments: C[0,33) G[33,97) G[97,146) C[146,163) G[163,263) C[263,268)
    y = W.generate(w)
    y.q[0, 120:] += 1.0
    y.k[0, 120:] += 1.0
    y.v[0, 120:] += 1.0
    pert, _ = run_fwd(refresh_bits(y))
    b0, p0 = base.cpu(), pert.cpu()
    assert torch.equal(b0[0, :97], p0[0, :97])          # rows that end before token 120
    assert not torch.equal(b0[0, 97:120], p0[0, 97:120])  # image rows see their whole segment


def test_gen_image_hidden_from_later_rows():
    """Rows after a Gen Image do not depend on its tokens; its own rows do."""
    w = SMALL["gen_small"].replace(batch=1)
    x = W.generate(w)
    base, _ = run_fwd(x)
    # segments: C[0,33) GEN[33,97) C[97,114) GEN[114,214) C[214,219)
    y = W.generate(w)
    y.k[0, 33:97] += 1.0
    y.v[0, 33:97] += 1.0
    pert, _ = run_fwd(refresh_bits(y))
    b0, p0 = base.cpu(), pert.cpu()
    assert torch.equal(b0[0, :33], p0[0, :33])            # before it
    assert torch.equal(b0[0, 97:], p0[0, 97:])            # everything after it
    assert not torch.equal(b0[0, 33:97], p0[0, 33:97])    # its own rows


def planned(x, dev, prescaled):
    """classifier + prologue + ha_attn_fwd_planned, q prescaled by the prologue or not."""
    w = x.workload
    desc = desc_for(w, x.segments)
    desc.c.q_prescaled = int(prescaled)
    pro = prologue_for(w, dev)
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    ranges = torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda")
    lim = torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")
    B.ha_classify_tiles(desc, None, ranges, lim)
    qr, kr = dev["q"], dev["k"]
    if pro is not None or prescaled:
        pro = pro or B.PrologueDesc("none")
        pro.c.q_out_scale = B.ha_q_prescale(desc) if prescaled else 0.0
        qr, kr = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
        B.ha_qk_prologue(desc, pro, dev["q"], dev["k"], qr, kr)
    out = torch.empty_like(dev["q"])
    B.ha_attn_fwd_planned(desc, qr, kr, dev["v"], lim, ranges, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["edit_small", "f32_mixed"])
def test_deterministic_and_fwd_equals_planned(name):
    w = SMALL[name]
    x = W.generate(w)
    a, dev = run_fwd(x)
    b, _ = run_fwd(x, dev)
    assert torch.equal(a, b)
    # ha_attn_fwd writes a prescaled q to its workspace: the same as the planned path (with
    # one work item per query block, as the planned path has)
    with unsplit():
        a, _ = run_fwd(x, dev)
    assert torch.equal(planned(x, dev, True), a)
    # plain q through the planned path: a different kernel variant, same result
    compare(f64(planned(x, dev, False)), oracle.hot_path(x), w.dtype, name + " planned plain q")


@pytest.mark.parametrize("name", ["hd_small", "f32_mixed"])
def test_prologue_q_out_scale(name):
    w = SMALL[name]
    x = W.generate(w)
    dev = to_device(x)
    desc, pro = desc_for(w), prologue_for(w, dev)
    pro.c.q_out_scale = 0.37
    qo, ko = torch.empty_like(dev["q"]), torch.empty_like(dev["k"])
    B.ha_qk_prologue(desc, pro, dev["q"], dev["k"], qo, ko)
    torch.cuda.synchronize()
    q_ref, k_ref = oracle.prologue(x)
    tol = (lambda want: 2.0 ** -7 * np.abs(want) + 1e-6) if w.dtype == "bf16" else (
        lambda want: 1e-5 * np.abs(want).max())
    assert (np.abs(f64(qo) - 0.37 * q_ref) <= tol(0.37 * q_ref)).all()
    assert (np.abs(f64(ko) - k_ref) <= tol(k_ref)).all()


@pytest.mark.parametrize("alpha,sign", [(16.0, 1.0), (26.0, 1.0), (36.0, -1.0)])
@pytest.mark.parametrize("prescaled", [False, True])
def test_extreme_logits(alpha, sign, prescaled):
    """q and k share a strong common direction e_0, which shifts every score of a row by
    about sign * alpha^2 * scale * log2(e): +33, +86 or -165 in log2 units for alpha 16, 26
    and 36 at head dim 128, so the softmax itself stays well conditioned. +33 stays on the
    fast path with huge P values; +86 (tile sums beyond 2^64) and -165 (every exp2
    underflows, even as a denormal) force the careful re-referencing pass. (A prescaled q
    is rounded after the scale, so its error grows with the common component.)"""
    w = small([W.Segment(C, 40), W.Segment(F, 100), W.Segment(G, 61)], rope="none", norm=False,
              hq=8, hkv=2)
    x = W.generate(w)
    x.q[..., 0] += sign * alpha
    x.k[..., 0] += alpha
    refresh_bits(x)
    dev = to_device(x)
    got = f64(planned(x, dev, prescaled))
    compare(got, oracle.hot_path(x), "bf16", f"extreme logits {sign * alpha} prescaled {prescaled}")


def test_extreme_logits_late_keys_one_head():
    """Only query head 3 and only keys from 130 on carry the common direction: the rows of
    that head leave the range at their third key tile, after two ordinary tiles, while
    every other head of the work item stays in range; the whole work item is redone on the
    careful pass and must still match."""
    w = small([W.Segment(C, 40), W.Segment(F, 100), W.Segment(G, 61)], rope="none", norm=False,
              hq=8, hkv=2)
    x = W.generate(w)
    x.q[:, :, 3, 0] += 26.0
    x.k[:, 130:, :, 0] += 26.0
    refresh_bits(x)
    dev = to_device(x)
    for prescaled in (False, True):
        got = f64(planned(x, dev, prescaled))
        compare(got, oracle.hot_path(x), "bf16", f"late extreme keys, one head, prescaled {prescaled}")


def test_per_batch_layouts_differ():
    w = small([W.Segment(C, 40), W.Segment(F, 60), W.Segment(G, 28)], batch=3)
    seg = W.segment_table(w)
    seg[1] = [[0, 100, F], [100, 10, C], [110, 18, G]]
    seg[2] = [[0, 1, C], [1, 64, G], [65, 63, G]]
    x = W.generate(w)
    x.segments = seg
    out, _ = run_fwd(x)
    compare(f64(out), oracle.hot_path(x), "bf16", "per-batch layouts")


def test_empty_inputs_launch_nothing():
    for b, s in ((0, 100), (2, 0)):
        desc = B.AttnDesc(b, s, 8, 2, 128, "bf16", np.zeros((b, 1, 3)) if b else [])
        B.ha_attn_fwd(desc, None, None, None, None, None, None, 0)
        B.ha_classify_tiles(desc, ranges=torch.empty(1, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()


def test_api_layer_matches_abi():
    w = SMALL["hd_small"]
    x = W.generate(w)
    ref, dev = run_fwd(x)
    cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len)
    out = api.hybrid_attention(dev["q"], dev["k"], dev["v"], x.segments, rope=w.rope,
                               positions=dev["positions"], cos_sin=cs,
                               mrope_sections=w.mrope_sections, q_norm_weight=dev["w_q"],
                               k_norm_weight=dev["w_k"], eps=w.norm_eps)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
