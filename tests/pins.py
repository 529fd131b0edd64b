"""Oracle pins: each function raises AssertionError when the oracle disagrees with
something other than itself (closed forms, library routines, invariants the pages fix,
brute force on tiny inputs). Used by test_oracle_*.py and, with mistakes planted in the
oracle, by test_oracle_mutations.py."""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
import oracle.masked_attention
import oracle.mask
import oracle.norm
import oracle.pipeline
import oracle.rope
import workloads as W
from oracle.brute import brute_force

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
C, F, G, GEN = W.SEG_CAUSAL, W.SEG_FULL, W.SEG_GCA, W.SEG_GEN


def small_workload(segs, hq=4, hkv=2, d=16, rope="mrope", sections=(4, 2, 2), norm=True,
                   batch=1, seed=7, theta=1e4, dtype="f32"):
    return W.Workload(name="small", description="small", batch=batch, segments=tuple(segs),
                      n_q_heads=hq, n_kv_heads=hkv, head_dim=d, dtype=dtype, rope=rope,
                      rope_theta=theta, mrope_sections=sections, qk_norm=norm, norm_eps=1e-6,
                      seed=seed)


def closed_form_pairs(segments, S):
    """Allowed pairs from arithmetic series, one term per segment: a causal segment
    [a, a+L) contributes sum_{i=a}^{a+L-1} (i+1); a full one L*S; an image (GCA or Gen
    Image) segment L*(a+L), since each of its rows sees every key before the segment end.
    Then each Gen Image [a, a+L) is removed from the S - (a+L) rows after it: every one of
    those rows would otherwise see all L of its keys (they all lie below the row)."""
    total = 0
    for a, L, kind in segments:
        a, L = int(a), int(L)
        if kind == C:
            total += L * a + L * (L + 1) // 2
        elif kind == F:
            total += L * S
        else:
            total += L * (a + L)
    for a, L, kind in segments:
        if kind == GEN:
            total -= int(L) * (S - int(a) - int(L))
    return total


# ---------------------------------------------------------------- mask
def pin_pair_counts():
    gold = json.load(open(os.path.join(GOLDEN, "pair_counts.json")))["counts"]
    for name, w in W.CONFIGS.items():
        table = W.segment_table(w)[0]
        got = oracle.mask.explicit_mask(table, w.seq_len).sum()
        assert got == closed_form_pairs(table, w.seq_len), name
        assert got == gold[name]["allowed_pairs_per_batch_item"], name


def pin_mask_elementwise_bruteforce():
    from oracle.brute import _allowed
    layouts = [[(C, 5), (F, 7), (C, 4)], [(C, 3), (G, 6), (C, 2), (G, 5), (G, 3), (C, 1)],
               [(G, 9)], [(F, 4), (C, 6)],
               [(C, 3), (GEN, 5), (C, 2), (GEN, 4), (F, 3), (C, 2)], [(GEN, 6), (C, 3)],
               [(C, 2), (GEN, 4), (GEN, 3), (G, 3), (C, 1)], [(F, 3), (GEN, 4), (F, 2)]]
    for segs in layouts:
        w = small_workload([W.Segment(k, n) for k, n in segs])
        table = W.segment_table(w)[0]
        M = oracle.mask.explicit_mask(table, w.seq_len)
        for i in range(w.seq_len):
            for j in range(w.seq_len):
                assert M[i, j] == _allowed(table, i, j), (segs, i, j)


def pin_mask_special_cases():
    S = 37
    tril = np.tril(np.ones((S, S), dtype=bool))
    t = np.array([[0, S, C]])
    assert np.array_equal(oracle.mask.explicit_mask(t, S), tril)
    for kind in (F, G):
        assert oracle.mask.explicit_mask(np.array([[0, S, kind]]), S).all()
    # the first text row attends only to itself
    t = np.array([[0, 10, C], [10, 27, F]])
    M = oracle.mask.explicit_mask(t, S)
    assert M[0, 0] and not M[0, 1:].any()
    # every row is a key prefix [0, lim), with lim > i (no empty row)
    t = np.array([[0, 5, C], [5, 9, G], [14, 3, C], [17, 12, G], [29, 8, F]])
    M = oracle.mask.explicit_mask(t, S)
    for i in range(S):
        lim = M[i].sum()
        assert lim > i and M[i, :lim].all() and not M[i, lim:].any()
    # merging adjacent causal or full segments changes nothing; splitting an image does
    a = oracle.mask.explicit_mask(np.array([[0, 10, C], [10, 27, C]]), S)
    assert np.array_equal(a, tril)
    b = oracle.mask.explicit_mask(np.array([[0, 20, G], [20, 17, G]]), S)
    assert not np.array_equal(b, oracle.mask.explicit_mask(np.array([[0, S, G]]), S))


def pin_mask_gen_hole():
    """Gen Images (multi-image training, HunyuanImage 3.0 digest, Figure 4(b)): the mask
    differs from the plain image (GCA) mask only by holes below the diagonal, one block
    [end, S) x [start, end) per Gen Image; its own rows see all of it; every row still
    sees itself; and with a single Gen Image at the end of the sequence (the inference
    case) the mask is the canonical GCA mask."""
    rng = np.random.default_rng(11)
    for trial in range(30):
        S = int(rng.integers(4, 60))
        n = int(rng.integers(1, 7))
        cuts = sorted(rng.choice(np.arange(1, S), size=min(S - 1, n - 1), replace=False).tolist())
        b = [0, *cuts, S]
        t = np.array([[a, e - a, int(rng.choice([C, F, G, GEN, GEN]))] for a, e in zip(b, b[1:])])
        M = oracle.mask.explicit_mask(t, S)
        as_gca = t.copy()
        as_gca[as_gca[:, 2] == GEN, 2] = G
        M_gca = oracle.mask.explicit_mask(as_gca, S)
        diff = M_gca & ~M
        assert not (M & ~M_gca).any()                 # only removes pairs
        assert not np.triu(diff).any()                # strictly below the diagonal
        hole = np.zeros((S, S), dtype=bool)
        for a, L, k in t:
            if k == GEN:
                hole[a + L:, a:a + L] = True
                assert M[a:a + L, a:a + L].all()      # the image's own rows see it
        assert np.array_equal(diff, hole), t.tolist()
        assert np.diagonal(M).all()
    t = np.array([[0, 7, C], [7, 9, G], [16, 5, C], [21, 12, GEN]])
    g = t.copy()
    g[3, 2] = G
    assert np.array_equal(oracle.mask.explicit_mask(t, 33), oracle.mask.explicit_mask(g, 33))


# ---------------------------------------------------------------- RMSNorm
def pin_rmsnorm_library():
    rng = np.random.default_rng(3)
    for scale in (1.0, 1e-3):   # small inputs make eps matter
        x = rng.standard_normal((5, 7, 3, 64)) * scale
        w = 1 + 0.02 * rng.standard_normal(64)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w),
                                           eps=1e-6).numpy()
        got = oracle.norm.rms_norm(x, w, 1e-6)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-15), scale


def pin_rmsnorm_closed_form():
    # d = 4, x = (3, 4, 0, 0): mean square 25/4, so with eps 0, y = x / 2.5 * w
    y = oracle.norm.rms_norm(np.array([3.0, 4.0, 0.0, 0.0]), np.array([1.0, 2.0, 3.0, 4.0]), 0.0)
    assert np.allclose(y, [1.2, 3.2, 0.0, 0.0], rtol=0, atol=1e-15)
    # with unit weights the output mean square is ms / (ms + eps)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((100, 32)) * 0.01
    eps = 1e-4
    y = oracle.norm.rms_norm(x, np.ones(32), eps)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)
    assert np.array_equal(oracle.norm.rms_norm(np.zeros(8), np.ones(8), 1e-6), np.zeros(8))


# ---------------------------------------------------------------- rotary
def _rot(x, pos, kind, sections=(0, 0, 0), base=1e4):
    d = x.shape[-1]
    axes = oracle.rope.axis_of_pair(kind, d, sections)
    ang = oracle.rope.rope_angles(pos, axes, oracle.rope.inv_freq(base, d))
    return oracle.rope.apply_rope(x, ang)


def pin_rope_reduces_to_1d():
    """2D (and 3-axis) rotary with every axis equal to n is 1D rotary at n, bit for bit
    (HunyuanImage 3.0 digest: with no image tokens the encoding reduces exactly to 1D)."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 50, 3, 128))
    n = rng.integers(0, 9000, size=(2, 50))
    one = _rot(x, n[..., None], "1d")
    assert np.array_equal(_rot(x, np.repeat(n[..., None], 2, -1), "2d"), one)
    assert np.array_equal(_rot(x, np.repeat(n[..., None], 3, -1), "mrope", (24, 20, 20), 5e6),
                          _rot(x, n[..., None], "1d", base=5e6))


def pin_rope_relative_position():
    """Scores depend on the position difference only (HunyuanImage 3.0 digest, 1D RoPE
    property), per axis for the multi-axis forms."""
    rng = np.random.default_rng(6)
    for kind, A, sec in (("1d", 1, (0, 0, 0)), ("2d", 2, (0, 0, 0)), ("mrope", 3, (24, 20, 20))):
        q = rng.standard_normal((1, 20, 1, 128))
        k = rng.standard_normal((1, 20, 1, 128))
        p = rng.integers(0, 3000, size=(1, 20, A))
        s0 = np.einsum("bihd,bjhd->ij", _rot(q, p, kind, sec), _rot(k, p, kind, sec))
        for a in range(A):
            shift = np.zeros(A, dtype=np.int64)
            shift[a] = 1234
            s1 = np.einsum("bihd,bjhd->ij", _rot(q, p + shift, kind, sec),
                           _rot(k, p + shift, kind, sec))
            assert np.abs(s1 - s0).max() < 1e-9 * np.abs(s0).max(), (kind, a)


def pin_rope_rotation_forms():
    """Rotate-half rotary equals multiplying z_i = x_i + i*x_{i+d/2} by exp(i*angle_i);
    it preserves the norm; position 0 is the identity."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 30, 2, 64))
    pos = rng.integers(0, 500, size=(1, 30, 2))
    y = _rot(x, pos, "2d")
    axes = np.arange(32) % 2
    ang = pos[..., axes].astype(np.float64) * 1e4 ** (-np.arange(32) / 32.0)
    z = (x[..., :32] + 1j * x[..., 32:]) * np.exp(1j * ang)[:, :, None, :]
    assert np.allclose(y[..., :32], z.real, atol=1e-12) and np.allclose(y[..., 32:], z.imag,
                                                                         atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(_rot(x, np.zeros_like(pos), "2d"), x)


def pin_rope_tables():
    gold = json.load(open(os.path.join(GOLDEN, "page_shapes.json")))
    sec = tuple(gold["mrope_sections"])
    axes = oracle.rope.axis_of_pair("mrope", gold["head_dim"], sec)
    assert [int((axes == a).sum()) for a in range(3)] == list(sec)
    # interleaved: the first 60 pairs cycle T, H, W; the rest are T
    assert list(axes[:6]) == [0, 1, 2, 0, 1, 2] and (axes[60:] == 0).all()
    assert list(oracle.rope.axis_of_pair("2d", 8)) == [0, 1, 0, 1]
    f = oracle.rope.inv_freq(5e6, 128)
    assert f[0] == 1.0 and np.allclose(f[1:] / f[:-1], 5e6 ** (-2 / 128), rtol=1e-13)
    assert len(f) == 64


# ---------------------------------------------------------------- attention
def _sdpa(q, k, v, mask=None, causal=False):
    """torch CPU fp64 scaled_dot_product_attention on [S][H][d] inputs (K/V per q head)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(np.transpose(a, (1, 0, 2))))
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=am,
                                                         is_causal=causal)
    return np.transpose(o.numpy(), (1, 0, 2))


def pin_attention_library():
    rng = np.random.default_rng(9)
    S, H, d = 61, 3, 32
    q, k, v = (rng.standard_normal((1, S, H, d)) for _ in range(3))
    # pure text: causal attention (BASELINE property; digest: text tokens are causal)
    M = oracle.mask.explicit_mask(np.array([[0, S, C]]), S)
    got = oracle.masked_attention.attention(q, k, v, [M])
    assert np.allclose(got[0], _sdpa(q[0], k[0], v[0], causal=True), atol=1e-12)
    # all-full: unmasked attention
    M = oracle.mask.explicit_mask(np.array([[0, S, F]]), S)
    got = oracle.masked_attention.attention(q, k, v, [M])
    assert np.allclose(got[0], _sdpa(q[0], k[0], v[0]), atol=1e-12)
    # hybrid mask passed to the library as a boolean mask
    M = oracle.mask.explicit_mask(np.array([[0, 9, C], [9, 20, G], [29, 7, C], [36, 25, F]]), S)
    got = oracle.masked_attention.attention(q, k, v, [M], row_chunk=16)
    assert np.allclose(got[0], _sdpa(q[0], k[0], v[0], mask=M), atol=1e-12)


def pin_attention_gqa():
    """GQA with 4 query heads per KV head equals MHA on K/V repeated per query head."""
    rng = np.random.default_rng(10)
    S = 33
    q = rng.standard_normal((1, S, 8, 16))
    k = rng.standard_normal((1, S, 2, 16))
    v = rng.standard_normal((1, S, 2, 16))
    M = oracle.mask.explicit_mask(np.array([[0, 11, C], [11, 22, F]]), S)
    gqa = oracle.masked_attention.attention(q, k, v, [M])
    for h in range(8):
        ref = _sdpa(q[0, :, h:h + 1], k[0, :, h // 4:h // 4 + 1], v[0, :, h // 4:h // 4 + 1],
                    mask=M)
        assert np.allclose(gqa[0, :, h:h + 1], ref, atol=1e-12), h


def pin_attention_invariants():
    rng = np.random.default_rng(11)
    w = small_workload([W.Segment(C, 6), W.Segment(G, 9), W.Segment(C, 4), W.Segment(F, 5)],
                       rope="2d", sections=(0, 0, 0))
    x = W.generate(w)
    out = oracle.pipeline.hot_path(x)
    # row 0 sees only itself: its output is v_0 of its KV head
    assert np.array_equal(out[0, 0], x.v[0, 0][np.arange(4) // 2])
    # a causal row does not depend on later tokens; an image row depends on its own
    # segment's later tokens but not on tokens past the segment end
    def perturb(i0, i1):
        y = W.generate(w)
        y.q[0, i0:i1] += 1.0
        y.k[0, i0:i1] += 1.0
        y.v[0, i0:i1] += 1.0
        return oracle.pipeline.hot_path(y)
    o2 = perturb(16, 24)                      # tokens 16.. : after text row 5, after image
    assert np.array_equal(o2[0, :15], out[0, :15])
    o3 = perturb(14, 15)                      # last token of the image segment [6, 15)
    assert not np.allclose(o3[0, 6], out[0, 6])
    assert np.array_equal(o3[0, :6], out[0, :6])
    # uniform probe: q = 0 gives uniform weights over the allowed prefix, so with one-hot
    # values the output is the fraction of allowed keys per value channel
    y = W.generate(w)
    y.q[:] = 0.0
    y.v[:] = 0.0
    S, d = w.seq_len, w.head_dim
    for j in range(S):
        y.v[0, j, :, j % d] = 1.0
    o4 = oracle.pipeline.hot_path(y)
    lims = {0: lambda i: i + 1}
    for i in range(S):
        lim = int(oracle.mask.mask_rows(y.segments[0], S, [i])[0].sum())
        expect = np.zeros(d)
        for j in range(lim):
            expect[j % d] += 1.0 / lim
        assert np.allclose(o4[0, i, 0], expect, atol=1e-14), i


def pin_bruteforce():
    cases = [W.get_config("tiny"),
             small_workload([W.Segment(C, 7), W.Segment(F, 9, (3, 3)), W.Segment(C, 4, (2, 2))],
                            rope="mrope", sections=(4, 2, 2), norm=True, batch=2),
             small_workload([W.Segment(C, 5), W.Segment(G, 6, (2, 3)), W.Segment(C, 3),
                             W.Segment(G, 4, (2, 2)), W.Segment(C, 2)], rope="2d", norm=False,
                            hq=2, hkv=1, d=8)]
    for w in cases:
        x = W.generate(w)
        assert np.abs(np.array(brute_force(x)) - oracle.pipeline.hot_path(x)).max() < 1e-12, w.name


# ---------------------------------------------------------------- tiles
def closed_form_labels(segments, S, bq, bk, q_end_aligned=False):
    """Labels from per-row key limits: a causal row i sees [0, i+1), a full row [0, S),
    an image row [0, end of its segment). Without Gen Images every row is a prefix, so per
    query block tiles below floor(min lim / bk) are FULL (all of them if min lim = S),
    tiles from ceil(max lim / bk) on are SKIP, and the rest PARTIAL. A Gen Image's keys
    are seen only by rows before its end (kvis = that end; S for other keys), so pair
    (i, j) is allowed iff j < lim(i) and i < kvis(j): a tile is FULL iff every row's
    limit covers it and every key's kvis lies past the block's last row, and SKIP when
    no row's limit reaches it or every key's kvis is at or before the block's first row
    (exact for these segment kinds). Query blocks start at row 0, or at S - nq * bq
    (clipped at 0) when end-aligned."""
    lim = np.empty(S, dtype=np.int64)
    kvis = np.full(S, S, dtype=np.int64)
    for a, L, kind in segments:
        i = np.arange(a, a + L)
        lim[a:a + L] = i + 1 if kind == C else (S if kind == F else a + L)
        if kind == GEN:
            kvis[a:a + L] = a + L
    nq, nk = -(-S // bq), -(-S // bk)
    q0 = S - nq * bq if q_end_aligned else 0
    out = np.empty((nq, nk), dtype=np.uint8)
    for qb in range(nq):
        r0, r1 = max(q0 + qb * bq, 0), min(q0 + (qb + 1) * bq, S)
        l = lim[r0:r1]
        for kb in range(nk):
            c0, c1 = kb * bk, min((kb + 1) * bk, S)
            kv = kvis[c0:c1]
            if l.max() <= c0 or kv.max() <= r0:
                out[qb, kb] = 0
            elif l.min() >= c1 and kv.min() > r1 - 1:
                out[qb, kb] = 1
            else:
                out[qb, kb] = 2
    return out


def pin_tile_labels():
    gold = json.load(open(os.path.join(GOLDEN, "tile_counts.json")))
    for name, w in W.CONFIGS.items():
        table = W.segment_table(w)[0]
        M = oracle.mask.explicit_mask(table, w.seq_len)
        for end in (False, True):
            for bq, bk in ((64, 64), (128, 64), (32, 64), (96, 64)):
                lab = oracle.tile_labels(M, bq, bk, q_end_aligned=end)
                want = closed_form_labels(table, w.seq_len, bq, bk, q_end_aligned=end)
                assert np.array_equal(lab, want), (name, bq, end)
            key = "counts_q_end_aligned" if end else "counts"
            lab = oracle.tile_labels(M, 64, 64, q_end_aligned=end)
            assert [int((lab == t).sum()) for t in (0, 1, 2)] == [
                gold[key][name]["skip"], gold[key][name]["full"], gold[key][name]["partial"]], name
    # random layouts of every kind, Gen Images included, at several block shapes
    rng = np.random.default_rng(12)
    for trial in range(60):
        S = int(rng.integers(2, 200))
        n = int(rng.integers(1, 8))
        cuts = sorted(rng.choice(np.arange(1, S), size=min(S - 1, n - 1), replace=False).tolist())
        b = [0, *cuts, S]
        t = np.array([[a, e - a, int(rng.choice([C, F, G, GEN, GEN]))] for a, e in zip(b, b[1:])])
        M = oracle.mask.explicit_mask(t, S)
        for bq, bk in ((64, 64), (128, 64), (16, 8), (8, 16)):
            assert np.array_equal(oracle.tile_labels(M, bq, bk, q_end_aligned=True),
                                  closed_form_labels(t, S, bq, bk, q_end_aligned=True)), (t.tolist(), bq)

# ---------------------------------------------------------------- QKV projection (oracle/projection.py)
def pin_projection_permutation():
    """A permutation weight picks input channels: y[..., i] = x[..., perm[i]] exactly, so
    q, k, v are known slices of x. Catches a transposed weight (which applies the inverse
    permutation) and a wrong order of the q, k and v sections."""
    w = small_workload([W.Segment(C, 6)], hq=4, hkv=2, d=8, rope="none", norm=False, batch=2)
    n_out = (w.n_q_heads + 2 * w.n_kv_heads) * w.head_dim
    rng = np.random.default_rng(5)
    perm = rng.permutation(n_out)
    P = np.zeros((n_out, n_out))
    P[np.arange(n_out), perm] = 1.0
    x = rng.standard_normal((w.batch, w.seq_len, n_out))
    q, k, v = oracle.qkv_projection(x, P, w.n_q_heads, w.n_kv_heads, w.head_dim)
    y = x[..., perm]
    nq, nkv = w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    assert np.array_equal(q, y[..., :nq].reshape(q.shape))
    assert np.array_equal(k, y[..., nq:nq + nkv].reshape(k.shape))
    assert np.array_equal(v, y[..., nq + nkv:].reshape(v.shape))


def pin_projection_bruteforce():
    """Scalar loops for the product, then the scalar norm and rotary of oracle/brute.py, per
    head: equal to the vectorised projection + prologue to rounding."""
    from oracle.brute import _axis_list, _prep
    for rope, sections in (("mrope", (2, 1, 1)), ("2d", (0, 0, 0))):
        w = small_workload([W.Segment(C, 3), W.Segment(F, 4, (2, 2))], hq=2, hkv=1, d=8, rope=rope,
                           sections=sections, norm=True, seed=9)
        x_in = W.generate(w)
        proj = W.generate_projection(w, hidden=12)
        q_rot, k_rot, v = oracle.qkv_prologue(x_in, proj.x, proj.w_qkv)
        axes = _axis_list(w.rope, w.head_dim // 2, w.mrope_sections)
        d = w.head_dim
        for t in range(w.seq_len):
            y = [sum(float(proj.x[0, t, c]) * float(proj.w_qkv[n, c]) for c in range(12))
                 for n in range(proj.w_qkv.shape[0])]
            pos = x_in.positions[0, t]
            for h in range(w.n_q_heads):
                want = _prep(y[h * d:(h + 1) * d], w, x_in.w_q, pos, axes)
                assert np.allclose(q_rot[0, t, h], want, rtol=1e-12, atol=1e-12), (rope, t, h)
            base = w.n_q_heads * d
            for g in range(w.n_kv_heads):
                want = _prep(y[base + g * d:base + (g + 1) * d], w, x_in.w_k, pos, axes)
                assert np.allclose(k_rot[0, t, g], want, rtol=1e-12, atol=1e-12), (rope, t, g)
                vb = base + w.n_kv_heads * d
                assert np.allclose(v[0, t, g], y[vb + g * d:vb + (g + 1) * d], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- backward (oracle/backward.py)

def _bwd_layout(rope="mrope", norm=True, batch=1, seed=21):
    """Tiny layout with every segment kind: text, a 2x2 full (HiDream generation) block,
    a 2x2 image (GCA) block, more text."""
    segs = [W.Segment(C, 3), W.Segment(F, 4, (2, 2)), W.Segment(G, 4, (2, 2)), W.Segment(C, 2)]
    return small_workload(segs, hq=4, hkv=2, d=8, rope=rope, sections=(2, 1, 1), norm=norm,
                          batch=batch, seed=seed)


def pin_backward_finite_differences():
    """Brute force: central differences of the forward path (pinned on its own by the pins
    above) agree with the backward for entries of q, k, v and both norm weights."""
    import dataclasses
    import oracle.backward
    w = _bwd_layout(batch=2)
    x = W.generate(w)
    rng = np.random.default_rng(5)
    dout = rng.standard_normal((w.batch, w.seq_len, w.n_q_heads, w.head_dim))
    g = oracle.backward.path_backward(x, dout)

    def loss(name, arr):
        y = dataclasses.replace(x, **{name: arr})
        return float(np.sum(oracle.pipeline.hot_path(y) * dout))

    h = 1e-5
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("w_q", "dw_q"), ("w_k", "dw_k")):
        base = np.asarray(getattr(x, name), dtype=np.float64)
        for i in rng.choice(base.size, size=min(8, base.size), replace=False):
            up, dn = base.copy(), base.copy()
            up.flat[i] += h
            dn.flat[i] -= h
            num = (loss(name, up) - loss(name, dn)) / (2 * h)
            got = g[key].flat[i]
            assert abs(num - got) <= 1e-6 * max(1.0, abs(num)), (name, int(i), num, got)


def pin_backward_autograd():
    """torch autograd (fp64, CPU) through F.rms_norm, a rotation and F.scaled_dot_product_
    attention with the boolean mask gives the same gradients as the oracle's formulas."""
    import oracle.backward
    for rope, norm in (("mrope", True), ("2d", False), ("none", True)):
        w = _bwd_layout(rope=rope, norm=norm, seed=22)
        x = W.generate(w)
        B, S, Hq, d = x.q.shape
        grp = Hq // w.n_kv_heads
        rng = np.random.default_rng(6)
        dout = rng.standard_normal((B, S, Hq, d))
        T = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
        q, k, v = T(x.q), T(x.k), T(x.v)
        wq = T(x.w_q) if norm else None
        wk = T(x.w_k) if norm else None
        qn = torch.nn.functional.rms_norm(q, (d,), wq, w.norm_eps) if norm else q
        kn = torch.nn.functional.rms_norm(k, (d,), wk, w.norm_eps) if norm else k
        if rope != "none":
            axes = oracle.rope.axis_of_pair(rope, d, w.mrope_sections)
            ang = torch.tensor(oracle.rope.rope_angles(x.positions, axes,
                                                       oracle.rope.inv_freq(w.rope_theta, d)))
            c, s = torch.cos(ang)[:, :, None, :], torch.sin(ang)[:, :, None, :]
            rot = lambda t: torch.cat([t[..., :d // 2] * c - t[..., d // 2:] * s,
                                       t[..., d // 2:] * c + t[..., :d // 2] * s], dim=-1)
            qn, kn = rot(qn), rot(kn)
        M = torch.tensor(np.stack([oracle.mask.explicit_mask(x.segments[b], S) for b in range(B)]))
        o = torch.nn.functional.scaled_dot_product_attention(
            qn.transpose(1, 2), kn.repeat_interleave(grp, dim=2).transpose(1, 2),
            v.repeat_interleave(grp, dim=2).transpose(1, 2), attn_mask=M[:, None])
        (o.transpose(1, 2) * torch.from_numpy(dout)).sum().backward()
        g = oracle.backward.path_backward(x, dout)
        for name, t in (("dq", q), ("dk", k), ("dv", v), ("dw_q", wq), ("dw_k", wk)):
            if t is None:
                assert g[name] is None, (rope, name)
                continue
            assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), (rope, name)


def pin_backward_invariants():
    """Closed forms of the attention backward (no norm, no rotary):
    - softmax rows sum to 1, so summed over keys dV_g equals the group's summed dO and
      dZ sums to 0 in every row, which makes dK summed over keys 0;
    - a row with one allowed key has a constant softmax, so its dq is 0;
    - lse of an all-zero query row is log(number of allowed keys) (pair counts in closed form)."""
    import oracle.backward
    rng = np.random.default_rng(12)
    table = np.array([[0, 5, C], [5, 12, G], [17, 9, F], [26, 4, C]])
    S, Hq, Hkv, d = 30, 6, 2, 16
    q = rng.standard_normal((1, S, Hq, d))
    k = rng.standard_normal((1, S, Hkv, d))
    v = rng.standard_normal((1, S, Hkv, d))
    dout = rng.standard_normal((1, S, Hq, d))
    M = oracle.mask.explicit_mask(table, S)
    dq, dk, dv = oracle.backward.attention_backward(q, k, v, [M], dout)
    for g in range(Hkv):
        assert np.allclose(dk[0, :, g].sum(axis=0), 0.0, atol=1e-10), g
        want = dout[0, :, 3 * g:3 * g + 3].sum(axis=(0, 1))
        assert np.allclose(dv[0, :, g].sum(axis=0), want, atol=1e-10), g
    assert np.allclose(dq[0, 0], 0.0, atol=1e-14)  # row 0 of a causal start sees key 0 only
    q0 = q.copy()
    q0[0, :, 0] = 0.0
    lse = oracle.backward.attention_lse(q0, k, [M])
    counts = np.array([(i + 1) if (i < 5 or i >= 26) else (17 if i < 17 else S) for i in range(S)])
    assert np.allclose(lse[0, 0], np.log(counts), atol=1e-12)


# ---------------------------------------------------------------- sampled rows and KV groups
def _rows_layouts():
    """Small layouts covering every segment kind, every rotary kind, norm on and off,
    groups of 1, 4 and 8 query heads per KV head, two batch items."""
    return [
        small_workload([W.Segment(C, 9), W.Segment(F, 16, (4, 4)), W.Segment(C, 6)], hq=4, hkv=1,
                       d=16, rope="mrope", sections=(4, 2, 2), norm=True, batch=2, seed=31),
        small_workload([W.Segment(C, 5), W.Segment(G, 9, (3, 3)), W.Segment(C, 4),
                        W.Segment(G, 16, (4, 4)), W.Segment(C, 3)], hq=8, hkv=1, d=16, rope="2d",
                       norm=False, batch=2, seed=32),
        small_workload([W.Segment(C, 4), W.Segment(GEN, 9, (3, 3)), W.Segment(C, 3),
                        W.Segment(GEN, 4, (2, 2)), W.Segment(F, 4, (2, 2)), W.Segment(C, 2)],
                       hq=4, hkv=4, d=8, rope="1d", norm=True, batch=2, seed=33),
        small_workload([W.Segment(G, 6, (2, 3)), W.Segment(C, 7), W.Segment(F, 9, (3, 3))], hq=8,
                       hkv=2, d=16, rope="none", norm=True, batch=2, seed=34),
    ]


def pin_rows_match_whole_path():
    """hot_path_rows (the checker of every full-size GPU test) equals the whole-path oracle,
    pinned on its own by the pins above, on sampled rows and heads of each batch item:
    both run the same norm, rotary and softmax, one on a subset of rows and heads."""
    rng = np.random.default_rng(35)
    for w in _rows_layouts():
        x = W.generate(w)
        whole = oracle.pipeline.hot_path(x)
        S, Hq = w.seq_len, w.n_q_heads
        for b in range(w.batch):
            for trial in range(3):
                n = int(rng.integers(1, S))
                rows = rng.choice(S, size=n, replace=False)
                if trial == 0:
                    rows = np.concatenate([[S - 1, 0], rows[:max(0, n - 2)]])
                heads = rng.choice(Hq, size=int(rng.integers(1, Hq + 1)), replace=False)
                got = oracle.pipeline.hot_path_rows(x, b, rows, list(heads))
                want = whole[b][rows][:, heads]
                assert got.shape == want.shape, (w.name, b)
                assert np.abs(got - want).max() <= 1e-12, (b, rows.tolist(), heads.tolist())


def pin_heads_match_whole_path():
    """hot_path restricted to some query heads (the checker of the full-size GPU tests that
    compare one KV group's heads whole) equals the whole call's entries for those heads, and
    leaves every other head unset."""
    rng = np.random.default_rng(37)
    for w in _rows_layouts():
        x = W.generate(w)
        whole = oracle.pipeline.hot_path(x)
        grp = w.n_q_heads // w.n_kv_heads
        for g in range(w.n_kv_heads):
            heads = list(range(g * grp, (g + 1) * grp))
            if rng.random() < 0.5:  # and an arbitrary subset
                heads = sorted(rng.choice(w.n_q_heads, size=int(rng.integers(1, w.n_q_heads + 1)),
                                          replace=False).tolist())
            part = oracle.pipeline.hot_path(x, heads=heads)
            assert np.abs(part[:, :, heads] - whole[:, :, heads]).max() <= 1e-12, (w.name, heads)
            others = [h for h in range(w.n_q_heads) if h not in heads]
            assert np.isnan(part[:, :, others]).all(), (w.name, heads)


def pin_backward_groups_match_whole():
    """path_backward restricted to some KV groups (the checker of the full-size backward
    GPU tests) equals the entries of the whole call, pinned by finite differences and torch
    autograd above, for those groups: dq of the group's query heads, dk and dv of the
    group; and it leaves every other entry unset."""
    import oracle.backward
    rng = np.random.default_rng(36)
    for w in _rows_layouts():
        x = W.generate(w)
        dout = rng.standard_normal((w.batch, w.seq_len, w.n_q_heads, w.head_dim))
        whole = oracle.backward.path_backward(x, dout)
        grp = w.n_q_heads // w.n_kv_heads
        for g in range(w.n_kv_heads):
            part = oracle.backward.path_backward(x, dout, groups=[g])
            hs = slice(g * grp, (g + 1) * grp)
            assert np.abs(part["dq"][:, :, hs] - whole["dq"][:, :, hs]).max() <= 1e-12, (w.name, g)
            assert np.abs(part["dk"][:, :, g] - whole["dk"][:, :, g]).max() <= 1e-12, (w.name, g)
            assert np.abs(part["dv"][:, :, g] - whole["dv"][:, :, g]).max() <= 1e-12, (w.name, g)
            others = [h for h in range(w.n_q_heads) if h // grp != g]
            assert np.isnan(part["dq"][:, :, others]).all(), (w.name, g)
            assert np.isnan(np.delete(part["dk"], g, axis=2)).all(), (w.name, g)
