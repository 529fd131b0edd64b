"""CPU oracle for hybrid-masked joint self-attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check of the package entry point and
the CPU-baseline leg of the benchmark may import or call anything in this package. The
product path (the HIP library and its Python binding) never imports it, and this package
never imports the product path. The two share no code; the only common module is the
seeded input generator in `workloads`, which holds none of the method's arithmetic.

What it computes, slowly and plainly, in float64 unless a function says otherwise:
  mask.py       explicit boolean mask from the segment-type rules
  norm.py       q/k RMSNorm
  rope.py       1D / generalized 2D / 3-axis interleaved rotary position embedding
  masked_attention.py  softmax(Q K^T * scale) V with the explicit mask, GQA head sharing
  tiles.py      tile labels SKIP / FULL / PARTIAL by brute force over the mask
  pipeline.py   the whole path in the pages' order: norm, rotary, mask, attention
  brute.py      scalar pure-Python fp64 re-derivation for tiny inputs
  backward.py   gradients of the whole path (attention, rotary, norm) and the row lse
  projection.py the QKV projection feeding the prologue (x W^T, split by heads, then norm
                and rotary)

Parity pins (tests/test_oracle_*.py) tie each part to something other than itself:
closed-form allowed-pair counts, library routines (torch CPU scaled_dot_product_attention
and rms_norm in fp64), the pages' stated special cases (pure text = causal attention,
2D rotary with no image = 1D rotary), invariants, and brute force on tiny inputs.
Parity unpinned (no worked example on the pages; only the stated reading is implemented):
which rotary pairs go to which axis in 2D and in mRoPE, the rotate-half pairing layout,
RMSNorm's eps placement and weight order, and the GQA head-to-group map.
"""
from .mask import segment_ids, mask_rows, explicit_mask, allowed_pairs
from .norm import rms_norm
from .rope import inv_freq, axis_of_pair, rope_angles, apply_rope
from .masked_attention import attention, attention_rows
from .tiles import tile_labels
from .pipeline import prologue, hot_path, hot_path_rows
from .backward import (attention_lse, attention_backward, rope_backward, rms_norm_backward,
                       path_lse, path_backward)
from .projection import qkv_projection, qkv_prologue

SEG_CAUSAL, SEG_FULL, SEG_GCA, SEG_GEN = 0, 1, 2, 3
LABEL_SKIP, LABEL_FULL, LABEL_PARTIAL = 0, 1, 2
