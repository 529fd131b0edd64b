"""Plant plausible mistakes in the oracle (CPU only) and check that a pin catches each.

Each case replaces one oracle function with a wrong variant (a dropped term, a wrong
sign, index or operand) and asserts that at least one of the listed pins fails."""
import numpy as np
import pytest

import oracle.backward
import oracle.mask
import oracle.masked_attention
import oracle.norm
import oracle.pipeline
import oracle.projection
import oracle.rope
import pins


def _rope_sign(x, angles, dtype=np.float64):
    x = np.asarray(x, dtype=dtype)
    h = x.shape[-1] // 2
    c = np.cos(angles)[:, :, None, :]
    s = np.sin(angles)[:, :, None, :]
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c - x[..., :h] * s], -1)


def _rope_adjacent_pairs(x, angles, dtype=np.float64):
    x = np.asarray(x, dtype=dtype)
    c = np.cos(angles)[:, :, None, :]
    s = np.sin(angles)[:, :, None, :]
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return y


def _inv_freq_half(base, d):
    return np.float64(base) ** (-np.arange(d // 2) / d)


def _axes_contiguous(kind, d, sections=(0, 0, 0)):
    if kind == "mrope":
        return np.repeat(np.arange(3), sections)
    return pins_axis(kind, d, sections)


pins_axis = oracle.rope.axis_of_pair


def _norm_eps_outside(x, w, eps, dtype=np.float64):
    x = np.asarray(x, dtype=dtype)
    return x / (np.sqrt(np.mean(x * x, -1, keepdims=True)) + eps) * w


def _norm_no_weight(x, w, eps, dtype=np.float64):
    x = np.asarray(x, dtype=dtype)
    return x / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)


def _norm_sum_not_mean(x, w, eps, dtype=np.float64):
    x = np.asarray(x, dtype=dtype)
    return x / np.sqrt(np.sum(x * x, -1, keepdims=True) + eps) * w


def _mask_strict_causal(segments, S, rows):
    M = _orig_mask_rows(segments, S, rows)
    table = np.asarray(segments)
    seg = oracle.mask.segment_ids(segments, S)
    for r, i in enumerate(np.asarray(rows)):
        if table[seg[i], 2] == 0 and i > 0:
            M[r, i] = False
    return M


def _mask_gca_no_segment(segments, S, rows):
    M = _orig_mask_rows(segments, S, rows)
    table = np.asarray(segments)
    seg = oracle.mask.segment_ids(segments, S)
    j = np.arange(S)
    for r, i in enumerate(np.asarray(rows)):
        if table[seg[i], 2] == 2:
            M[r] = j <= i
    return M


def _mask_gen_variant(strict=False, none=False, own_rows=False):
    """Gen Image hole mistakes: rows at the image's end still see it (strict), no hole at
    all (none), or the image hidden from its own rows too (own_rows)."""
    def mask_rows(segments, S, rows):
        table = np.asarray(segments)
        as_gca = table.copy()
        as_gca[as_gca[:, 2] == 3, 2] = 2
        M = _orig_mask_rows(as_gca, S, rows)
        if none:
            return M
        for r, i in enumerate(np.asarray(rows)):
            for a, L, k in table:
                if k == 3 and (i > a + L if strict else (i >= a if own_rows else i >= a + L)):
                    M[r, a:a + L] = False
        return M
    return mask_rows


def _proj_variant(transposed=False, kv_swapped=False):
    def qkv_projection(x, w_qkv, n_q_heads, n_kv_heads, head_dim, dtype=np.float64):
        x = np.asarray(x, dtype=dtype)
        w = np.asarray(w_qkv, dtype=dtype)
        B, S, _ = x.shape
        y = x @ w if transposed else x @ w.T
        nq, nkv = n_q_heads * head_dim, n_kv_heads * head_dim
        q = y[..., :nq].reshape(B, S, n_q_heads, head_dim)
        k = y[..., nq:nq + nkv].reshape(B, S, n_kv_heads, head_dim)
        v = y[..., nq + nkv:nq + 2 * nkv].reshape(B, S, n_kv_heads, head_dim)
        return (q, v, k) if kv_swapped else (q, k, v)
    return qkv_projection


_orig_mask_rows = oracle.mask.mask_rows
_orig_attention = oracle.masked_attention.attention


def _attn_no_scale(q, k, v, masks, scale=None, **kw):
    return _orig_attention(q, k, v, masks, scale=1.0, **kw)


def _attn_k_for_v(q, k, v, masks, scale=None, **kw):
    return _orig_attention(q, k, k, masks, scale=scale, **kw)


def _attn_gqa_modulo(q, k, v, masks, scale=None, dtype=np.float64, heads=None, row_chunk=1024):
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    out = np.empty((B, S, Hq, d))
    for h in range(Hq):
        g = h % Hkv
        out[:, :, h:h + 1] = _orig_attention(q[:, :, h:h + 1], k[:, :, g:g + 1], v[:, :, g:g + 1],
                                             masks, scale=(1 / np.sqrt(d)) if scale is None else scale)
    return out


def _attn_transposed_scores(q, k, v, masks, scale=None, dtype=np.float64, heads=None,
                            row_chunk=1024):
    B, S, Hq, d = q.shape
    group = Hq // k.shape[2]
    scale = 1 / np.sqrt(d) if scale is None else scale
    out = np.empty((B, S, Hq, d))
    for b in range(B):
        for h in range(Hq):
            Q, K, V = q[b, :, h], k[b, :, h // group], v[b, :, h // group]
            Z = np.where(masks[b], (K @ Q.T) * scale, -np.inf)
            Z = np.exp(Z - Z.max(-1, keepdims=True))
            out[b, :, h] = (Z / Z.sum(-1, keepdims=True)) @ V
    return out


MUTATIONS = {
    "rope_sign": ([(oracle.rope, "apply_rope", _rope_sign), (oracle.pipeline, "apply_rope", _rope_sign)],
                  ["pin_rope_rotation_forms"]),
    "rope_adjacent_pairs": ([(oracle.rope, "apply_rope", _rope_adjacent_pairs),
                             (oracle.pipeline, "apply_rope", _rope_adjacent_pairs)],
                            ["pin_rope_rotation_forms", "pin_bruteforce"]),
    "rope_freq_exponent": ([(oracle.rope, "inv_freq", _inv_freq_half),
                            (oracle.pipeline, "inv_freq", _inv_freq_half)],
                           ["pin_rope_tables", "pin_bruteforce"]),
    "mrope_contiguous_sections": ([(oracle.rope, "axis_of_pair", _axes_contiguous),
                                   (oracle.pipeline, "axis_of_pair", _axes_contiguous)],
                                  ["pin_rope_tables", "pin_bruteforce"]),
    "norm_eps_outside_sqrt": ([(oracle.norm, "rms_norm", _norm_eps_outside)],
                              ["pin_rmsnorm_library"]),
    "norm_no_weight": ([(oracle.norm, "rms_norm", _norm_no_weight),
                        (oracle.pipeline, "rms_norm", _norm_no_weight)],
                       ["pin_rmsnorm_library", "pin_rmsnorm_closed_form", "pin_bruteforce"]),
    "norm_sum_not_mean": ([(oracle.norm, "rms_norm", _norm_sum_not_mean)],
                          ["pin_rmsnorm_library", "pin_rmsnorm_closed_form"]),
    "mask_strict_causal": ([(oracle.mask, "mask_rows", _mask_strict_causal)],
                           ["pin_pair_counts", "pin_mask_special_cases",
                            "pin_mask_elementwise_bruteforce"]),
    "mask_gca_without_segment": ([(oracle.mask, "mask_rows", _mask_gca_no_segment)],
                                 ["pin_pair_counts", "pin_mask_special_cases"]),
    "mask_gen_hole_off_by_one": ([(oracle.mask, "mask_rows", _mask_gen_variant(strict=True))],
                                 ["pin_pair_counts", "pin_mask_gen_hole", "pin_mask_elementwise_bruteforce"]),
    "mask_gen_no_hole": ([(oracle.mask, "mask_rows", _mask_gen_variant(none=True))],
                         ["pin_pair_counts", "pin_mask_gen_hole", "pin_mask_elementwise_bruteforce"]),
    "mask_gen_hidden_from_itself": ([(oracle.mask, "mask_rows", _mask_gen_variant(own_rows=True))],
                                    ["pin_pair_counts", "pin_mask_gen_hole", "pin_mask_elementwise_bruteforce"]),
    "projection_transposed_weight": ([(oracle.projection, "qkv_projection", _proj_variant(transposed=True)),
                                      (oracle, "qkv_projection", _proj_variant(transposed=True))],
                                     ["pin_projection_permutation", "pin_projection_bruteforce"]),
    "projection_k_v_swapped": ([(oracle.projection, "qkv_projection", _proj_variant(kv_swapped=True)),
                                (oracle, "qkv_projection", _proj_variant(kv_swapped=True))],
                               ["pin_projection_permutation", "pin_projection_bruteforce"]),
    "attn_dropped_scale": ([(oracle.masked_attention, "attention", _attn_no_scale)],
                           ["pin_attention_library"]),
    "attn_k_used_as_v": ([(oracle.masked_attention, "attention", _attn_k_for_v)],
                         ["pin_attention_library"]),
    "attn_gqa_modulo_map": ([(oracle.masked_attention, "attention", _attn_gqa_modulo)],
                            ["pin_attention_gqa"]),
    "attn_transposed_scores": ([(oracle.masked_attention, "attention", _attn_transposed_scores)],
                               ["pin_attention_library"]),
}


# ---- backward (oracle/backward.py)
def _bwd_variant(no_delta=False, overwrite_dv=False, unscaled_dk=False, untransposed_dz=False):
    def attention_backward(q, k, v, masks, dout, scale=None, groups=None):
        q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
        B, S, Hq, d = q.shape
        Hkv = k.shape[2]
        group = Hq // Hkv
        scale = (1.0 / np.sqrt(d)) if scale is None else scale
        dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(B):
            for g in range(Hkv):
                K, V = k[b, :, g], v[b, :, g]
                for h in range(g * group, (g + 1) * group):
                    Q, dO = q[b, :, h], dout[b, :, h]
                    Z = np.where(masks[b], Q @ K.T * scale, -np.inf)
                    P = np.exp(Z - Z.max(-1, keepdims=True))
                    P /= P.sum(-1, keepdims=True)
                    dP = dO @ V.T
                    dZ = P * dP if no_delta else P * (dP - np.sum(dO * (P @ V), -1, keepdims=True))
                    if overwrite_dv:
                        dv[b, :, g] = P.T @ dO
                    else:
                        dv[b, :, g] += P.T @ dO
                    dq[b, :, h] = scale * dZ @ K
                    dk[b, :, g] += (1.0 if unscaled_dk else scale) * ((dZ if untransposed_dz else dZ.T) @ Q)
        return dq, dk, dv
    return attention_backward


def _rope_bwd_same_rotation(dy, angles):
    return oracle.rope.apply_rope(dy, np.asarray(angles, dtype=np.float64))


def _norm_bwd_first_term(x, weight, eps, dy):
    x, dy, w = (np.asarray(a, dtype=np.float64) for a in (x, dy, weight))
    r = 1.0 / np.sqrt(np.mean(x * x, -1, keepdims=True) + eps)
    return r * dy * w, np.sum((dy * x * r).reshape(-1, x.shape[-1]), axis=0)


_BWD_PINS = ["pin_backward_finite_differences", "pin_backward_autograd", "pin_backward_invariants"]
MUTATIONS.update({
    "bwd_softmax_without_delta": ([(oracle.backward, "attention_backward", _bwd_variant(no_delta=True))],
                                  _BWD_PINS),
    "bwd_dv_one_head_of_group": ([(oracle.backward, "attention_backward", _bwd_variant(overwrite_dv=True))],
                                 _BWD_PINS),
    "bwd_dk_without_scale": ([(oracle.backward, "attention_backward", _bwd_variant(unscaled_dk=True))],
                             _BWD_PINS[:2]),
    "bwd_dk_untransposed_dz": ([(oracle.backward, "attention_backward", _bwd_variant(untransposed_dz=True))],
                               _BWD_PINS),
    "bwd_rope_forward_rotation": ([(oracle.backward, "rope_backward", _rope_bwd_same_rotation)],
                                  _BWD_PINS[:2]),
    "bwd_norm_first_term_only": ([(oracle.backward, "rms_norm_backward", _norm_bwd_first_term)],
                                 _BWD_PINS[:2]),
})


# ---- sampled rows and KV-group subsets (the checkers of the full-size GPU tests)
def _rows_positions_by_item(inputs, b, rows, heads, dtype=np.float64):
    """hot_path_rows with the positions cut to the batch item but not to the sampled rows
    (the first len(rows) tokens' positions rotate the sampled q rows)."""
    w = inputs.workload
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(inputs.q[b:b + 1, rows], dtype=dtype)
    k = np.asarray(inputs.k[b:b + 1], dtype=dtype)
    if w.qk_norm:
        q = oracle.norm.rms_norm(q, inputs.w_q, w.norm_eps, dtype=dtype)
        k = oracle.norm.rms_norm(k, inputs.w_k, w.norm_eps, dtype=dtype)
    q = oracle.pipeline._rotary(q, w, inputs.positions[b:b + 1, :len(rows)], dtype)[0]
    k = oracle.pipeline._rotary(k, w, inputs.positions[b:b + 1], dtype)[0]
    mrows = oracle.mask.mask_rows(inputs.segments[b], w.seq_len, rows)
    return oracle.masked_attention.attention_rows(q, k, inputs.v[b], mrows, np.arange(len(rows)),
                                                  heads, dtype=dtype)


def _attention_rows_modulo_group(q, k, v, mask_rows, rows, heads, scale=None, dtype=np.float64):
    """attention_rows with KV head h mod Hkv instead of h div (Hq / Hkv)."""
    S, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = (1.0 / np.sqrt(d)) if scale is None else scale
    rows = np.asarray(rows)
    out = np.empty((len(rows), len(heads), d), dtype=dtype)
    for hi, h in enumerate(heads):
        g = h % Hkv
        Z = np.where(mask_rows, (q[rows, h, :] @ k[:, g, :].T) * scale, -np.inf)
        P = np.exp(Z - Z.max(-1, keepdims=True))
        out[:, hi, :] = (P / P.sum(-1, keepdims=True)) @ v[:, g, :]
    return out


_orig_attention_backward = oracle.backward.attention_backward


def _bwd_groups_enumerated(q, k, v, masks, dout, scale=None, groups=None):
    """attention_backward that takes the K and V of the i-th requested group from KV head i
    (right for a whole call, where the i-th group is group i; wrong for a subset)."""
    if groups is None:
        return _orig_attention_backward(q, k, v, masks, dout, scale=scale)
    Hkv = k.shape[2]
    order = list(groups)
    perm = list(range(Hkv))
    for i, g in enumerate(order):
        perm[g] = i
    kk = np.asarray(k)[:, :, perm]
    vv = np.asarray(v)[:, :, perm]
    return _orig_attention_backward(q, kk, vv, masks, dout, scale=scale, groups=groups)


MUTATIONS.update({
    "rows_positions_by_item_only": ([(oracle.pipeline, "hot_path_rows", _rows_positions_by_item)],
                                    ["pin_rows_match_whole_path"]),
    "rows_head_to_group_modulo": ([(oracle.masked_attention, "attention_rows", _attention_rows_modulo_group),
                                   (oracle.pipeline, "attention_rows", _attention_rows_modulo_group)],
                                  ["pin_rows_match_whole_path"]),
    "bwd_groups_enumerated_kv": ([(oracle.backward, "attention_backward", _bwd_groups_enumerated)],
                                 ["pin_backward_groups_match_whole"]),
})


_orig_attention = oracle.masked_attention.attention


def _attention_heads_enumerated(q, k, v, masks, scale=None, dtype=np.float64, heads=None, row_chunk=1024):
    """heads= mistake: the i-th requested query head reads the KV head of its place in the
    list (i // group) instead of its own (h // group)."""
    if heads is None:
        return _orig_attention(q, k, v, masks, scale=scale, dtype=dtype, row_chunk=row_chunk)
    heads = list(heads)
    group = q.shape[2] // k.shape[2]
    out = np.full(q.shape, np.nan, dtype=dtype)
    for i, h in enumerate(heads):
        kk, vv = np.array(k, copy=True), np.array(v, copy=True)
        src = min(i // group, k.shape[2] - 1)
        kk[:, :, h // group] = k[:, :, src]
        vv[:, :, h // group] = v[:, :, src]
        out[:, :, h] = _orig_attention(q, kk, vv, masks, scale=scale, dtype=dtype, heads=[h],
                                       row_chunk=row_chunk)[:, :, h]
    return out


MUTATIONS.update({
    "heads_subset_enumerated_kv": ([(oracle.pipeline, "attention", _attention_heads_enumerated)],
                                   ["pin_heads_match_whole_path"]),
})


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    patches, pin_names = MUTATIONS[name]
    for mod, attr, fn in patches:
        monkeypatch.setattr(mod, attr, fn)
    caught = []
    for p in pin_names:
        try:
            getattr(pins, p)()
        except (AssertionError, ValueError, IndexError):
            caught.append(p)
    assert caught, f"mutation {name} passed every pin in {pin_names}"
