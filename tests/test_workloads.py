"""The synthetic inputs have the shapes the pages give, and the generator is deterministic."""
import json
import os

import numpy as np

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_page_sequence_lengths():
    gold = json.load(open(os.path.join(GOLDEN, "page_shapes.json")))
    pc = W.page_shape_configs()
    assert pc["page1024"].seq_len == gold["sequence_lengths"]["1024x1024"]
    assert pc["page2048"].seq_len == gold["sequence_lengths"]["2048x2048"]
    p = gold["patch_pixels"]
    assert (1024 // p) ** 2 == 1024 and (2048 // p) ** 2 == 4096
    for name in ("hd1024", "hd2048", "edit"):
        w = W.get_config(name)
        assert (w.n_q_heads, w.n_kv_heads, w.head_dim) == (
            gold["gqa_q_heads"], gold["gqa_kv_heads"], gold["head_dim"])
        assert w.mrope_sections == tuple(gold["mrope_sections"])
        assert w.rope_theta == gold["mrope_theta"]


def test_hunyuan_grid():
    gold = json.load(open(os.path.join(GOLDEN, "hunyuan_shapes.json")))
    w = W.get_config("hunyuan")
    assert any(s.length == gold["image_1024_tokens"] and s.grid == tuple(gold["image_1024_grid"])
               for s in w.segments)


def test_config_sizes():
    want = {"tiny": 80, "hd1024": 1282, "hd2048": 4354, "edit": 8448, "hunyuan": 6016,
            "hunyuan_multigen": 6016}
    assert {n: c.seq_len for n, c in W.CONFIGS.items()} == want


def test_positions_recipe():
    w = W.get_config("hunyuan")
    pos = W.positions_for(w)[0]
    # text on the diagonal
    assert (pos[:512] == np.arange(512)[:, None]).all()
    # image A starts at 512 with a 32x32 grid: (x, y) = (512 + col, 512 + row)
    assert tuple(pos[512]) == (512, 512) and tuple(pos[512 + 33]) == (513, 513)
    assert tuple(pos[512 + 31]) == (543, 512)
    # image coordinates lie between the surrounding text positions
    img = pos[512:1536]
    assert img.min() > 511 and img.max() < 1536
    w3 = W.get_config("hd2048")
    p3 = W.positions_for(w3)[0]
    assert tuple(p3[258]) == (258, 258, 258) and tuple(p3[258 + 64 + 5]) == (258, 259, 263)
    assert p3.max() < w3.seq_len


def test_generator_deterministic_and_rounded():
    w = W.get_config("tiny")
    a, b = W.generate(w), W.generate(w)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    small = W.Workload(name="s", description="", batch=1, segments=(W.Segment(0, 8),),
                       n_q_heads=2, n_kv_heads=1, head_dim=8, dtype="bf16", rope="1d",
                       rope_theta=1e4, seed=3)
    x = W.generate(small)
    assert np.array_equal(W.bf16_bits_to_f32(x.q_bits), x.q)
    assert (x.q.view(np.uint32) & 0xFFFF == 0).all()
    # ties to even: 0x3f808000 -> 0x3f80 (even), 0x3f818000 -> 0x3f82 (odd rounds up)
    t = np.array([1.00390625, 1.005859375, 1.01171875], dtype=np.float32)
    assert list(W.f32_to_bf16_bits(t)) == [0x3F80, 0x3F81, 0x3F82]


def test_segment_table():
    t = W.segment_table(W.get_config("edit"))
    assert t.shape == (2, 3, 3)
    assert t[0].tolist() == [[0, 256, 0], [256, 4096, 1], [4352, 4096, 0]]
