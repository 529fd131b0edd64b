"""Workload table: the sequence layouts the pages describe, as concrete shapes.

Segment kinds (the per-token segment type of the unified sequence):
  SEG_CAUSAL  text, marker, condition and reference tokens: causal rows
              (HiDream-O1 atlas page, "How it works"; hidream-o1-p100a model card,
              "What this model is"; HunyuanImage 3.0 digest, "Generalized Causal
              Attention", text tokens).
  SEG_FULL    HiDream-O1 generation patches: rows attend to the whole sequence
              (same two HiDream pages).
  SEG_GCA     HunyuanImage 3.0 image segment: rows attend to everything before them
              plus every token of their own segment (HunyuanImage 3.0 digest,
              "Generalized Causal Attention", the core rule).
  SEG_GEN     HunyuanImage 3.0 Gen Image of a multi-image training sequence: rows as
              SEG_GCA, and no token after the segment attends to it (same digest,
              "Generalized Causal Attention", the multi-generation training paragraph).

Shapes: HiDream-O1 uses 32x32-pixel patches, so a 1024^2 image is a 32x32 grid and
2048^2 is 64x64, behind a chat-template prefix that ends in the two markers
<|boi|><|tms|>; batch 2 stands for the conditional and unconditional forwards of
CFG 5.0 (model card, "What this model is" and the Performance table). The backbone
is GQA 32/8 with head dim 128, q/k RMSNorm and 3-axis interleaved mRoPE [24,20,20]
at theta 5e6 (model card, architecture paragraph). HunyuanImage 3.0 interleaves text
and image segments and uses generalized 2D RoPE on images, 1D RoPE on text
(HunyuanImage 3.0 digest, "Generalized 2D Rotary Position Embedding").
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

SEG_CAUSAL = 0
SEG_FULL = 1
SEG_GCA = 2
SEG_GEN = 3

ROPE_NONE = "none"
ROPE_1D = "1d"
ROPE_2D = "2d"
ROPE_MROPE = "mrope"


@dataclass(frozen=True)
class Segment:
    kind: int
    length: int
    grid: Optional[Tuple[int, int]] = None  # (rows, cols) for image segments

    def __post_init__(self):
        if self.grid is not None and self.grid[0] * self.grid[1] != self.length:
            raise ValueError("grid does not match segment length")


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    batch: int
    segments: Tuple[Segment, ...]
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "bf16" or "f32": storage/compute type of q, k, v, out
    rope: str                  # one of ROPE_*
    rope_theta: float
    mrope_sections: Tuple[int, int, int] = (0, 0, 0)
    qk_norm: bool = False
    norm_eps: float = 1e-6
    seed: int = 0

    @property
    def seq_len(self) -> int:
        return sum(s.length for s in self.segments)

    @property
    def n_axes(self) -> int:
        return {ROPE_NONE: 1, ROPE_1D: 1, ROPE_2D: 2, ROPE_MROPE: 3}[self.rope]

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _hd(name, desc, batch, segs, seed, **kw):
    base = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", rope=ROPE_MROPE,
                rope_theta=5e6, mrope_sections=(24, 20, 20), qk_norm=True, norm_eps=1e-6)
    base.update(kw)
    return Workload(name=name, description=desc, batch=batch, segments=tuple(segs), seed=seed,
                    **base)


C, F, G, GEN = SEG_CAUSAL, SEG_FULL, SEG_GCA, SEG_GEN

CONFIGS = {
    "tiny": Workload(
        name="tiny",
        description="fp32 check: 16 causal text + 64 full generation tokens (8x8), "
                    "GQA 4/1, d=64, 1D RoPE on text and 2D (row, col) on patches, theta 1e4",
        batch=1, segments=(Segment(C, 16), Segment(F, 64, (8, 8))),
        n_q_heads=4, n_kv_heads=1, head_dim=64, dtype="f32", rope=ROPE_2D,
        rope_theta=1e4, qk_norm=False, seed=0),
    "hd1024": _hd("hd1024", "HiDream-O1-style 1024^2 t2i: B=2, 258 causal (256 text + 2 "
                  "markers) + 1024 full (32x32), GQA 32/8, d=128, bf16",
                  2, [Segment(C, 258), Segment(F, 1024, (32, 32))], seed=1),
    "hd2048": _hd("hd2048", "HiDream-O1-style 2048^2 t2i: B=2, 258 causal (256 text + 2 "
                  "markers) + 4096 full (64x64), GQA 32/8, d=128, bf16",
                  2, [Segment(C, 258), Segment(F, 4096, (64, 64))], seed=2),
    "edit": _hd("edit", "editing layout: B=2, 256 causal text + 4096 full generation "
                "(64x64) + 4096 causal reference (64x64), GQA 32/8, d=128, bf16",
                2, [Segment(C, 256), Segment(F, 4096, (64, 64)), Segment(C, 4096, (64, 64))],
                seed=3),
    "hunyuan": Workload(
        name="hunyuan",
        description="HunyuanImage-style generalized causal interleave: B=1, [512 text]"
                    "[1024 image 32x32][256 text][4096 image 64x64][128 text], GQA 32/8, "
                    "d=128, bf16, 2D RoPE on images, 1D on text, theta 1e4",
        batch=1,
        segments=(Segment(C, 512), Segment(G, 1024, (32, 32)), Segment(C, 256),
                  Segment(G, 4096, (64, 64)), Segment(C, 128)),
        n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", rope=ROPE_2D,
        rope_theta=1e4, qk_norm=False, seed=4),
    "hunyuan_multigen": Workload(
        name="hunyuan_multigen",
        description="HunyuanImage-style multi-image training sequence: B=1, [512 text]"
                    "[1024 Gen Image 32x32][256 text][4096 Gen Image 64x64][128 text], every "
                    "Gen Image hidden from the tokens after it, GQA 32/8, d=128, bf16, 2D RoPE "
                    "on images, 1D on text, theta 1e4",
        batch=1,
        segments=(Segment(C, 512), Segment(GEN, 1024, (32, 32)), Segment(C, 256),
                  Segment(GEN, 4096, (64, 64)), Segment(C, 128)),
        n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16", rope=ROPE_2D,
        rope_theta=1e4, qk_norm=False, seed=6),
}


def get_config(name: str) -> Workload:
    return CONFIGS[name]


def page_shape_configs():
    """Batch-1 shapes with the model card's own sequence lengths (Performance table):
    1050 tokens at 1024^2 and 4122 at 2048^2, i.e. a 26-token text+marker prefix before
    a 32x32 or 64x64 patch grid. Context shapes, not gating."""
    return {
        "page1024": _hd("page1024", "model-card 1024^2 shape: B=1, 26 causal + 1024 full",
                        1, [Segment(C, 26), Segment(F, 1024, (32, 32))], seed=11),
        "page2048": _hd("page2048", "model-card 2048^2 shape: B=1, 26 causal + 4096 full",
                        1, [Segment(C, 26), Segment(F, 4096, (64, 64))], seed=12),
    }
