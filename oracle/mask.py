"""Explicit boolean attention mask from per-token segment types.

Rules, one per segment kind, taken row by row as the pages state them:
  CAUSAL (0)  text, markers, condition and reference tokens attend to the tokens before
              them and to themselves: M[i, j] = j <= i.
              HiDream-O1 atlas page, "How it works" (condition and text tokens are
              causally masked); hidream-o1-p100a model card, "What this model is" (text
              tokens attend causally); HunyuanImage 3.0 digest, "Generalized Causal
              Attention" (text tokens attend only to previous tokens).
              Reading: "preceding" includes the token itself; otherwise row 0 would have
              no key at all.
  FULL (1)    HiDream-O1 generation tokens attend to everything: M[i, j] = True.
              Same two HiDream pages.
  GCA (2)     HunyuanImage 3.0 image tokens attend to every earlier token and to every
              token of their own image segment:
              M[i, j] = (j <= i) or (segment(j) == segment(i)).
              HunyuanImage 3.0 digest, "Generalized Causal Attention", the core rule;
              HunyuanImage 3.0 summary page, "Key claims".
  GEN (3)     a Gen Image of a multi-image HunyuanImage 3.0 training sequence (one that is
              being denoised while later tokens follow it): its own rows follow the GCA
              rule, and no token after it attends to it, so the mask gets a hole below the
              diagonal: M[i, j] = False for j in a GEN segment that ends at or before i,
              whatever the kind of row i. HunyuanImage 3.0 digest, "Generalized Causal
              Attention", the multi-generation training complication and Figure 4(b).
              Reading: "subsequent tokens" are the tokens after the segment's end, so the
              image's own rows keep seeing it; later Gen Images are subsequent tokens too.
Adjacent GCA segments are distinct images and are not merged.
"""
from __future__ import annotations

import numpy as np


def segment_ids(segments: np.ndarray, seq_len: int) -> np.ndarray:
    """Segment index of every token, from one batch item's (start, length, kind) rows."""
    seg = np.full(seq_len, -1, dtype=np.int64)
    for idx, (start, length, _kind) in enumerate(np.asarray(segments)):
        seg[start:start + length] = idx
    if (seg < 0).any():
        raise ValueError("segment table does not cover the sequence")
    return seg


def mask_rows(segments: np.ndarray, seq_len: int, rows) -> np.ndarray:
    """bool [len(rows)][S]; row r is query token rows[r]; True where it may attend to j."""
    S = seq_len
    seg = segment_ids(segments, S)
    table = np.asarray(segments)
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(S)
    M = np.zeros((len(rows), S), dtype=bool)
    for r, i in enumerate(rows):
        idx = seg[i]
        kind = table[idx, 2]
        if kind == 0:
            M[r] = j <= i
        elif kind == 1:
            M[r] = True
        elif kind in (2, 3):
            M[r] = (j <= i) | (seg == idx)
        else:
            raise ValueError(f"unknown segment kind {kind}")
        # the hole: Gen Images that ended at or before token i
        for start, length, kind_g in table:
            if kind_g == 3 and start + length <= i:
                M[r, start:start + length] = False
    return M


def explicit_mask(segments: np.ndarray, seq_len: int) -> np.ndarray:
    """bool [S][S]; True where query row i may attend to key column j."""
    return mask_rows(segments, seq_len, np.arange(seq_len))


def allowed_pairs(segments: np.ndarray, seq_len: int) -> int:
    return int(explicit_mask(segments, seq_len).sum())
