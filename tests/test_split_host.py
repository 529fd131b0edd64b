"""The split planner of the bf16 forward, on the host (no GPU, no kernel launched).

ha_attn_workspace_bytes grows by the plan's work item table and fp32 partial results exactly
when the planner splits query blocks, so the workspace size shows its decisions. The CU count
comes from the descriptor's plan_cus (without a device, and without it, nothing is split);
split_parts = 1 disables the plan and split_parts = P splits every block into P parts."""
import numpy as np
import pytest

import unified_text_pixel_amd as U
import workloads as W


def r256(n):
    return (n + 255) // 256 * 256


def wdesc(name):
    w = W.get_config(name)
    return U.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype,
                      W.segment_table(w))


def nbytes(d, split_parts=0, plan_cus=0):
    """Workspace bytes with the descriptor's split_parts and plan_cus set as given."""
    old = (d.c.split_parts, d.c.plan_cus)
    try:
        d.c.split_parts, d.c.plan_cus = int(split_parts), int(plan_cus)
        return U.ha_attn_workspace_bytes(d)
    finally:
        d.c.split_parts, d.c.plan_cus = old


def plan_bytes(d, n_items, n_splits, n_slots):
    """Workspace bytes a plan adds: the item and split tables (16 bytes an entry), then per
    slot the partial output [BQ][G][d] and the row sums and references [BQ][G], fp32."""
    bq = U.ha_tile_shape(d)[0]
    g = d.c.n_q_heads // d.c.n_kv_heads
    per = n_slots * bq * g
    return r256((n_items + n_splits) * 16) + r256(per * d.c.head_dim * 4) + 2 * r256(per * 4)


def test_no_cu_count_no_split():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a device is present: its CU count drives the planner")
    except ImportError:
        pass
    for name in ("hunyuan", "hd1024"):
        d = wdesc(name)
        assert nbytes(d) == nbytes(d, split_parts=1)


def test_hunyuan_on_256_cus():
    """Each XCD serves one (batch, KV head) pair: 94 query blocks, of which 66 are heavy (the
    64 blocks of the 64x64 image, 92 key tiles, and the last 2 text blocks, 93 and 94). 64 of
    them fill 2 rounds of 32 CUs; the other 2 are split into 4 parts each: 100 items per XCD,
    16 split blocks in all, 64 partial slots."""
    d = wdesc("hunyuan")
    base = nbytes(d, split_parts=1)
    assert nbytes(d, plan_cus=256) - base == plan_bytes(d, 800, 16, 64)


@pytest.mark.parametrize("name,cus,split", [("hd2048", 256, False), ("edit", 256, False),
                                            ("hunyuan_multigen", 256, False),
                                            ("hunyuan_multigen", 240, True), ("hd2048", 240, True),
                                            ("hunyuan", 192, False)])
def test_planner_decisions(name, cus, split):
    """hd2048's 64 generation blocks per pair fill 4 whole rounds and edit gains under 3%;
    hunyuan_multigen's heaviest blocks skip the first Gen Image (76 tiles) and fill 2 rounds;
    on 30 CUs per XCD they leave 4 over, which are split."""
    d = wdesc(name)
    base = nbytes(d, split_parts=1)
    got = nbytes(d, plan_cus=cus)
    assert (got > base) == split, (name, cus, got - base)


def test_forced_parts():
    """split_parts = 3: every (KV head, query block) in 3 parts, whatever the CU count."""
    d = U.AttnDesc(1, 80, 8, 2, 128, "bf16", np.array([[[0, 16, 0], [16, 64, 1]]], np.int32))
    nq = U.ha_tile_shape(d)[2]
    blocks = 1 * 2 * nq
    base = nbytes(d, split_parts=1)
    for cus in (8, 256):
        assert nbytes(d, split_parts=3, plan_cus=cus) - base == plan_bytes(d, 3 * blocks, blocks,
                                                                               3 * blocks)


def test_fp32_never_split():
    d = U.AttnDesc(1, 80, 4, 1, 64, "f32", np.array([[[0, 16, 0], [16, 64, 1]]], np.int32))
    assert nbytes(d, split_parts=4, plan_cus=8) == nbytes(d, split_parts=1)


def test_per_batch_layouts_pad_the_table():
    """Item 0 ([100 causal][900 full]) and item 1 ([700 causal][300 image]) on 4 KV heads:
    each XCD plans one (item, KV head) pair, so the two items' lists differ in length (item
    0's heavy full-row blocks are split, item 1's causal blocks are not) and the table pads
    them to the longest: 22 entries per XCD, 176 in all, 12 split blocks, 36 slots."""
    seg = np.array([[[0, 100, 0], [100, 900, 1]], [[0, 700, 0], [700, 300, 2]]], np.int32)
    d = U.AttnDesc(2, 1000, 16, 4, 128, "bf16", seg)
    base = nbytes(d, split_parts=1)
    assert nbytes(d, plan_cus=96) - base == plan_bytes(d, 176, 12, 36)
