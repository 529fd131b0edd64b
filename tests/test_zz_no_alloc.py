"""ha_attn_fwd_static: the forward without a caller workspace, for callers that cannot
allocate (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc). Its
scratch is a fixed device array of the library. Checked through the C ABI against
ha_attn_fwd (no prologue, with a workspace) on two calls in a row, the second smaller, with
a split plan and Gen Image holes among them; a problem too large for the array is refused
before any launch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import compare, desc_for, f64, require_gpu
from test_gpu_parity import SMALL
from unified_text_pixel_amd import HAError, binding as B
from workloads.device import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(w, x=None):
    """(static output, workspace output, inputs) for plain q, k (no prologue)."""
    x = W.generate(w) if x is None else x
    dev = to_device(x)
    desc = desc_for(w, x.segments)
    ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, None)), dtype=torch.uint8, device="cuda")
    ref = torch.full_like(dev["q"], float("nan"))
    B.ha_attn_fwd(desc, None, dev["q"], dev["k"], dev["v"], ref, ws)
    got = torch.full_like(dev["q"], float("nan"))
    B.ha_attn_fwd_static(desc, dev["q"], dev["k"], dev["v"], got)
    torch.cuda.synchronize()
    return got, ref, x


@pytest.mark.parametrize("first,second", [("hunyuan", "gca_small"), ("hunyuan_multigen", "gen_small"),
                                          ("hd2048", "hd_small")])
def test_static_matches_workspace_entry_point(first, second):
    """Two calls in a row: a full-size layout (the HunyuanImage ones take the split plan on
    256 CUs, the multi-image one the Gen Image tile lists), then a smaller one whose scratch
    contents are left over from the first. Each is bitwise equal to ha_attn_fwd on the same
    inputs (same kernels, same plan), and the small one matches the oracle."""
    w1 = W.get_config(first).replace(rope="none", qk_norm=False)
    got, ref, _ = _both(w1)
    assert torch.equal(got, ref), first
    w2 = SMALL[second].replace(rope="none", qk_norm=False)
    got, ref, x = _both(w2)
    assert torch.equal(got, ref), second
    compare(f64(got), oracle.hot_path(x), w2.dtype, f"static after {first}: {second}")


def test_static_fp32_and_forced_split():
    w = SMALL["f32_mixed"].replace(rope="none", qk_norm=False)
    got, ref, x = _both(w)
    assert torch.equal(got, ref)
    compare(f64(got), oracle.hot_path(x), "f32", "static fp32")
    w = SMALL["edit_small"].replace(rope="none", qk_norm=False)
    x = W.generate(w)
    dev = to_device(x)
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments,
                      split_parts=3)
    out = torch.empty_like(dev["q"])
    B.ha_attn_fwd_static(desc, dev["q"], dev["k"], dev["v"], out)
    torch.cuda.synchronize()
    compare(f64(out), oracle.hot_path(x), "bf16", "static, every block in 3 parts")


def test_static_refuses_problems_beyond_the_array():
    """Row limits alone need 4 bytes a token: 8 items of 600,000 tokens need more than
    the 16 MiB array, which is refused on the host (the device pointers are never used)."""
    S = 600_000
    desc = B.AttnDesc(8, S, 8, 2, 128, "bf16", np.array([[[0, S, 0]]] * 8, np.int32))
    fake = 1 << 20
    with pytest.raises(HAError) as e:
        B.ha_attn_fwd_static(desc, fake, fake, fake, fake)
    assert e.value.status == B.HA_ERR_WORKSPACE and "static array holds" in str(e.value)
