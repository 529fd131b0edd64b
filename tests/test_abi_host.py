"""C-ABI library on the host, no GPU: it loads, exports what include/ha_attn.h declares,
and rejects every invalid call with the right status before any HIP call (the device
pointers below are never dereferenced: validation fails first)."""
import os
import re

import numpy as np
import pytest

import oracle
import unified_text_pixel_amd as U
from unified_text_pixel_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ha_attn.h")
FAKE = 1 << 20  # 16-byte aligned, never dereferenced in these tests


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:[A-Za-z_][A-Za-z0-9_]*[ *]+)+(ha_[a-z0-9_]+)\(", text,
                                 flags=re.M)))


def test_exports_every_declared_symbol():
    lib = U.load_library()
    names = declared_functions()
    assert len(names) == 17 and sorted(B.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n
    assert U.ha_abi_version() == 5


def seg(rows, batch=1):
    return np.array([rows] * batch, dtype=np.int32)


def desc(**kw):
    base = dict(batch=1, seq_len=80, n_q_heads=4, n_kv_heads=1, head_dim=64, dtype="f32",
                segments=seg([[0, 16, 0], [16, 64, 1]]))
    base.update(kw)
    return U.AttnDesc(**base)


BAD_DESCS = [
    (dict(n_q_heads=6, n_kv_heads=4), B.HA_ERR_INVALID_ARG, "multiple"),
    (dict(n_q_heads=48, n_kv_heads=3), B.HA_ERR_UNSUPPORTED, "supported: 1, 2, 4, 8"),
    (dict(head_dim=96), B.HA_ERR_UNSUPPORTED, "head_dim"),
    (dict(dtype=7), B.HA_ERR_INVALID_ARG, "dtype"),
    (dict(scale=-1.0), B.HA_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), B.HA_ERR_INVALID_ARG, "scale"),
    (dict(seq_len=79, segments=seg([[0, 16, 0], [16, 64, 1]])), B.HA_ERR_SEGMENTS, "cover"),
    (dict(segments=seg([[0, 16, 0], [17, 63, 1]])), B.HA_ERR_SEGMENTS, "starts at"),
    (dict(segments=seg([[0, 16, 0], [16, 0, 1], [16, 64, 1]])), B.HA_ERR_SEGMENTS, "length"),
    (dict(segments=seg([[0, 16, 0], [16, 64, 5]])), B.HA_ERR_SEGMENTS, "kind"),
    (dict(segments=seg([[0, -4, 0], [-4, 84, 1]])), B.HA_ERR_SEGMENTS, "length"),
    (dict(seq_len=(1 << 22) + 1, segments=seg([[0, (1 << 22) + 1, 0]])), B.HA_ERR_UNSUPPORTED,
     "exceeds"),
    (dict(batch=-1), B.HA_ERR_INVALID_ARG, ">= 0"),
    (dict(n_kv_heads=0), B.HA_ERR_INVALID_ARG, "head counts"),
    (dict(q_prescaled=2), B.HA_ERR_INVALID_ARG, "q_prescaled"),
    (dict(split_parts=-1), B.HA_ERR_INVALID_ARG, "split_parts"),
    (dict(split_parts=65), B.HA_ERR_INVALID_ARG, "split_parts"),
    (dict(plan_cus=-3), B.HA_ERR_INVALID_ARG, "plan_cus"),
]


@pytest.mark.parametrize("kw,status,text", BAD_DESCS)
def test_bad_descriptor_rejected_everywhere(kw, status, text):
    d = desc(**kw)
    calls = [
        lambda: U.ha_tile_shape(d),
        lambda: U.ha_classify_tiles(d, ranges=FAKE, stream=0),
        lambda: U.ha_attn_fwd_planned(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
        lambda: U.ha_attn_fwd(d, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0),
        lambda: U.ha_qk_prologue(d, U.PrologueDesc("none"), FAKE, FAKE, FAKE, FAKE, stream=0),
        lambda: U.ha_attn_fwd_lse(d, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0),
        lambda: U.ha_attn_fwd_planned_from(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, stream=0),
        lambda: U.ha_qk_prologue_from(d, U.PrologueDesc("none"), FAKE, FAKE, FAKE, FAKE, 0, stream=0),
        lambda: U.ha_attn_bwd(d, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                              FAKE, 1 << 30, stream=0),
        lambda: U.ha_qkv_prologue(d, None, FAKE, 256, FAKE, FAKE, FAKE, FAKE, stream=0),
        lambda: U.ha_attn_fwd_static(d, FAKE, FAKE, FAKE, FAKE, stream=0),
    ]
    for call in calls:
        with pytest.raises(U.HAError) as e:
            call()
        assert e.value.status == status and text in str(e.value), str(e.value)
    assert U.ha_attn_workspace_bytes(d) == 0
    assert U.ha_attn_bwd_workspace_bytes(d) == 0


def test_bad_pointers_and_workspace():
    d = desc()
    with pytest.raises(U.HAError) as e:
        U.ha_attn_fwd_planned(d, None, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.HA_ERR_INVALID_ARG
    with pytest.raises(U.HAError) as e:
        U.ha_attn_fwd_planned(d, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.HA_ERR_ALIGNMENT
    need = U.ha_attn_workspace_bytes(d)
    assert need > 0 and need % 256 == 0
    for ws, nbytes in ((None, need), (FAKE + 16, need), (FAKE, need - 1)):
        with pytest.raises(U.HAError) as e:
            U.ha_attn_fwd(d, None, FAKE, FAKE, FAKE, FAKE, ws, nbytes, stream=0)
        assert e.value.status == B.HA_ERR_WORKSPACE
    with pytest.raises(U.HAError) as e:
        U.ha_classify_tiles(d, stream=0)
    assert e.value.status == B.HA_ERR_INVALID_ARG


BAD_PROLOGUES = [
    (dict(rope_kind=9), B.HA_ERR_INVALID_ARG, "rope_kind"),
    (dict(rope_kind="2d", positions=None, cos_sin=FAKE, n_pos=80), B.HA_ERR_INVALID_ARG, "required"),
    (dict(rope_kind="2d", positions=FAKE, cos_sin=FAKE, n_pos=0), B.HA_ERR_INVALID_ARG, "n_pos"),
    (dict(rope_kind="2d", positions=FAKE + 2, cos_sin=FAKE, n_pos=8), B.HA_ERR_ALIGNMENT, "misaligned"),
    (dict(rope_kind="mrope", positions=FAKE, cos_sin=FAKE, n_pos=8, mrope_sections=(24, 20, 20)),
     B.HA_ERR_INVALID_ARG, "sum to 32"),
    (dict(rope_kind="none", q_norm_weight=FAKE), B.HA_ERR_INVALID_ARG, "both"),
    (dict(rope_kind="none", q_norm_weight=FAKE, k_norm_weight=FAKE, eps=-1.0),
     B.HA_ERR_INVALID_ARG, "eps"),
    (dict(rope_kind="none", q_norm_weight=FAKE + 1, k_norm_weight=FAKE), B.HA_ERR_ALIGNMENT,
     "aligned"),
    (dict(rope_kind="none", q_out_scale=-1.0), B.HA_ERR_INVALID_ARG, "q_out_scale"),
    (dict(rope_kind="none", q_out_scale=float("inf")), B.HA_ERR_INVALID_ARG, "q_out_scale"),
]


@pytest.mark.parametrize("kw,status,text", BAD_PROLOGUES)
def test_bad_prologue_rejected(kw, status, text):
    d = desc()
    p = U.PrologueDesc(**kw)
    for call in (lambda: U.ha_qk_prologue(d, p, FAKE, FAKE, FAKE, FAKE, stream=0),
                 lambda: U.ha_attn_fwd(d, p, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)):
        with pytest.raises(U.HAError) as e:
            call()
        assert e.value.status == status and text in str(e.value), str(e.value)


def test_prologue_block_limit():
    d = desc(n_q_heads=128, n_kv_heads=16, head_dim=128, segments=seg([[0, 80, 0]]))
    with pytest.raises(U.HAError) as e:
        U.ha_qk_prologue(d, U.PrologueDesc("none"), FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.HA_ERR_UNSUPPORTED


def test_empty_work_is_ok_without_launch():
    for kw in (dict(batch=0, segments=np.zeros((0, 0, 3))), dict(seq_len=0, segments=seg([]))):
        d = desc(**kw)
        U.ha_attn_fwd(d, None, None, None, None, None, None, 0, stream=0)
        U.ha_attn_fwd_planned(d, None, None, None, None, None, None, stream=0)
        U.ha_classify_tiles(d, ranges=FAKE, stream=0)
        assert U.ha_last_error() == ""


def test_error_text_cleared_by_success():
    with pytest.raises(U.HAError):
        U.ha_tile_shape(desc(head_dim=96))
    assert "head_dim" in U.ha_last_error()
    U.ha_tile_shape(desc())
    assert U.ha_last_error() == ""


def test_q_prescale():
    d = desc()
    assert abs(U.ha_q_prescale(d) - np.log2(np.e) / 8.0) < 1e-7
    assert abs(U.ha_q_prescale(desc(scale=0.5)) - 0.5 * np.log2(np.e)) < 1e-7
    assert U.ha_q_prescale(desc(head_dim=96)) == 0.0


def test_tile_shape():
    assert U.ha_tile_shape(desc()) == (32, 64, 3, 2)
    d = desc(batch=2, seq_len=4354, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
             segments=seg([[0, 258, 0], [258, 4096, 1]], 2))
    assert U.ha_tile_shape(d) == (64, 64, 69, 69)
    # bf16: eight waves of 32 rows over the G query heads of a KV head
    for g, bq in ((1, 256), (2, 128), (4, 64), (8, 32)):
        d = desc(n_q_heads=8, n_kv_heads=8 // g, dtype="bf16")
        assert U.ha_tile_shape(d)[0] == bq
    # fp32: four waves
    for g, bq in ((1, 128), (2, 64), (8, 32)):
        d = desc(n_q_heads=8, n_kv_heads=8 // g)
        assert U.ha_tile_shape(d)[0] == bq


def test_rope_table_matches_oracle_angles():
    for theta, d in ((1e4, 64), (5e6, 128)):
        t = U.ha_rope_table_fill(theta, d, 300)
        ang = np.arange(300, dtype=np.float64)[:, None] * oracle.inv_freq(theta, d)[None, :]
        assert np.allclose(t[..., 0], np.cos(ang), atol=1e-7, rtol=0)
        assert np.allclose(t[..., 1], np.sin(ang), atol=1e-7, rtol=0)
    with pytest.raises(U.HAError) as e:
        U.ha_rope_table_fill(1e4, 100, 10)
    assert e.value.status == B.HA_ERR_UNSUPPORTED
    with pytest.raises(U.HAError):
        U.ha_rope_table_fill(0.5, 64, 10)


def test_workspace_layout():
    d = desc(batch=2, seq_len=4354, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
             segments=seg([[0, 258, 0], [258, 4096, 1]], 2))
    plain = U.ha_attn_workspace_bytes(d)
    with_pro = U.ha_attn_workspace_bytes(d, U.PrologueDesc("none"))
    assert plain >= 2 * 4354 * 4 + 2 * 69 * 8
    assert with_pro - plain >= 2 * 4354 * 40 * 128 * 2


def bf16_desc(**kw):
    base = dict(batch=1, seq_len=80, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype="bf16",
                segments=seg([[0, 16, 0], [16, 64, 1]]))
    base.update(kw)
    return U.AttnDesc(**base)


def test_training_entry_points_reject_before_launch():
    F = FAKE
    bwd = lambda d, p=None, dwq=None, dwk=None, ws=F, n=1 << 30, lse=F: U.ha_attn_bwd(
        d, p, F, F, F, F, lse, F, F, F, F, dwq, dwk, ws, n, stream=0)
    cases = [
        # fp32 tensors and groups of 8 query heads per KV head have no training kernels
        (lambda: U.ha_attn_fwd_lse(desc(), None, F, F, F, F, F, F, 1 << 30, stream=0), B.HA_ERR_UNSUPPORTED, "bf16"),
        (lambda: bwd(desc()), B.HA_ERR_UNSUPPORTED, "bf16"),
        (lambda: bwd(bf16_desc(n_q_heads=16)), B.HA_ERR_UNSUPPORTED, "1, 2, 4"),
        (lambda: U.ha_attn_fwd_lse(bf16_desc(), None, F, F, F, F, None, F, 1 << 30, stream=0),
         B.HA_ERR_INVALID_ARG, "lse"),
        (lambda: bwd(bf16_desc(), lse=None), B.HA_ERR_INVALID_ARG, "lse"),
        (lambda: bwd(bf16_desc(q_prescaled=1)), B.HA_ERR_INVALID_ARG, "q_prescaled"),
        # weight gradients exactly when the prologue normalises
        (lambda: bwd(bf16_desc(), dwq=F, dwk=F), B.HA_ERR_INVALID_ARG, "dw_q"),
        (lambda: bwd(bf16_desc(), U.PrologueDesc("none", q_norm_weight=F, k_norm_weight=F)),
         B.HA_ERR_INVALID_ARG, "dw_q"),
        (lambda: bwd(bf16_desc(), ws=None), B.HA_ERR_WORKSPACE, "NULL"),
        (lambda: bwd(bf16_desc(), n=U.ha_attn_bwd_workspace_bytes(bf16_desc()) - 1), B.HA_ERR_WORKSPACE, "needs"),
    ]
    for call, status, text in cases:
        with pytest.raises(U.HAError) as e:
            call()
        assert e.value.status == status and text in str(e.value), str(e.value)


def test_backward_workspace_layout():
    d = bf16_desc(batch=2, seq_len=4354, n_q_heads=32, n_kv_heads=8,
                  segments=seg([[0, 258, 0], [258, 4096, 1]], 2))
    plain = U.ha_attn_bwd_workspace_bytes(d)
    normed = U.ha_attn_bwd_workspace_bytes(d, U.PrologueDesc("none", q_norm_weight=FAKE, k_norm_weight=FAKE))
    tokens = 2 * 4354
    # bf16 rebuilt q, k + fp32 gradients of both + per-row delta
    assert plain >= tokens * 40 * 128 * (2 + 4) + tokens * 32 * 4
    assert normed - plain >= 2 * tokens * 128 * 4


def test_prefix_entry_points_check_ranges():
    d = desc()
    for bad in (-1, 81):
        with pytest.raises(U.HAError) as e:
            U.ha_attn_fwd_planned_from(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bad, stream=0)
        assert e.value.status == B.HA_ERR_INVALID_ARG and "row_begin" in str(e.value)
        with pytest.raises(U.HAError) as e:
            U.ha_qk_prologue_from(d, U.PrologueDesc("none"), FAKE, FAKE, FAKE, FAKE, bad, stream=0)
        assert e.value.status == B.HA_ERR_INVALID_ARG and "token_begin" in str(e.value)
    # nothing left to compute: no launch, no error
    U.ha_attn_fwd_planned_from(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 80, stream=0)
    U.ha_qk_prologue_from(d, U.PrologueDesc("none"), FAKE, FAKE, FAKE, FAKE, 80, stream=0)
    assert U.ha_last_error() == ""


def test_prefix_entry_point_refuses_rows_that_see_later_keys():
    """ha_attn_fwd_planned_from keeps the rows below row_begin from an earlier step, so it
    refuses a row_begin below which some row attends to a key at or after it: inside or
    after the start of a full segment (its rows see every key), or inside an image segment
    (its rows see their whole segment). The check runs on the host, before any launch."""
    full = desc(segments=seg([[0, 16, 0], [16, 64, 1]], batch=2), batch=2)
    gca = desc(segments=seg([[0, 16, 0], [16, 32, 2], [48, 32, 0]]))
    for d, p in ((full, 17), (full, 40), (full, 79), (gca, 17), (gca, 47)):
        with pytest.raises(U.HAError) as e:
            U.ha_attn_fwd_planned_from(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, p, stream=0)
        assert e.value.status == B.HA_ERR_INVALID_ARG and "attend to keys at or after" in str(e.value), p
    # the same rule as the torch layer's check
    from unified_text_pixel_amd.api import prefix_is_invariant
    for d, p in ((full, 17), (gca, 20)):
        assert not prefix_is_invariant(d._seg_np, d.c.seq_len, p)


def test_gen_image_layouts():
    """Gen Image segments (kind 3) are accepted; the planned calls, which lack the hole
    plan, refuse them before any launch; the workspaces grow by the plan arrays."""
    g = seg([[0, 16, 0], [16, 32, 3], [48, 32, 0]])
    d = desc(segments=g)
    for call in (lambda: U.ha_attn_fwd_planned(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0),
                 lambda: U.ha_attn_fwd_planned_from(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, stream=0)):
        with pytest.raises(U.HAError) as e:
            call()
        assert e.value.status == B.HA_ERR_UNSUPPORTED and "Gen Image" in str(e.value)
    plain = desc(segments=seg([[0, 16, 0], [16, 32, 2], [48, 32, 0]]))
    _, _, nq, nk = U.ha_tile_shape(d)
    extra = 256 * 4 + nq * nk * 4 + nq * 2 * 4   # key visibility (rows padded to 256), lists, counts
    assert U.ha_attn_workspace_bytes(d) - U.ha_attn_workspace_bytes(plain) >= extra
    bd, bp = bf16_desc(segments=g), bf16_desc(segments=seg([[0, 16, 0], [16, 32, 2], [48, 32, 0]]))
    assert U.ha_attn_bwd_workspace_bytes(bd) - U.ha_attn_bwd_workspace_bytes(bp) >= extra


def test_qkv_projection_rejects_before_launch():
    bf = bf16_desc()
    cases = [
        (lambda: U.ha_qkv_prologue(desc(), None, FAKE, 256, FAKE, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_UNSUPPORTED, "bf16"),
        (lambda: U.ha_qkv_prologue(bf16_desc(head_dim=64), None, FAKE, 256, FAKE, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_UNSUPPORTED, "head_dim"),
        (lambda: U.ha_qkv_prologue(bf, None, FAKE, 100, FAKE, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_UNSUPPORTED, "multiple of 64"),
        (lambda: U.ha_qkv_prologue(bf, None, FAKE, 0, FAKE, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_UNSUPPORTED, "multiple of 64"),
        (lambda: U.ha_qkv_prologue(bf, None, None, 256, FAKE, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_INVALID_ARG, "x is NULL"),
        (lambda: U.ha_qkv_prologue(bf, None, FAKE, 256, FAKE + 8, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_ALIGNMENT, "w_qkv"),
        (lambda: U.ha_qkv_prologue(bf, U.PrologueDesc("2d"), FAKE, 256, FAKE, FAKE, FAKE, FAKE, stream=0),
         B.HA_ERR_INVALID_ARG, "required"),
    ]
    for call, status, text in cases:
        with pytest.raises(U.HAError) as e:
            call()
        assert e.value.status == status and text in str(e.value), str(e.value)
    # no tokens: nothing to do, no launch
    U.ha_qkv_prologue(bf16_desc(batch=0, segments=np.zeros((0, 0, 3))), None, None, 256, None, None, None, None,
                      stream=0)
    assert U.ha_last_error() == ""


def test_static_forward_rejects_before_launch():
    """ha_attn_fwd_static: bad pointers, and a problem whose scratch exceeds the library's
    16 MiB array (row limits alone: 4 bytes a token, 8 x 600,000 tokens), fail on the host."""
    with pytest.raises(U.HAError) as e:
        U.ha_attn_fwd_static(desc(), None, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.HA_ERR_INVALID_ARG and "q is NULL" in str(e.value)
    S = 600_000
    big = U.AttnDesc(8, S, 8, 2, 128, "bf16", np.array([[[0, S, 0]]] * 8, np.int32))
    with pytest.raises(U.HAError) as e:
        U.ha_attn_fwd_static(big, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == B.HA_ERR_WORKSPACE and "static array holds 16777216" in str(e.value)
    U.ha_attn_fwd_static(desc(batch=0, segments=np.zeros((0, 0, 3))), None, None, None, None, stream=0)
    assert U.ha_last_error() == ""
