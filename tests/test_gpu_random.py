"""Seeded random layouts, whole outputs against the oracle: the forward (bf16 and fp32, with
and without forced split parts) and the training backward. Each case draws the batch, a
per-item segment table with every kind (Gen Images included) and cut points anywhere
(ragged against the 64-key tiles), the head ratio, the head dim, the rotary form and q/k
norm; the same positions and tables feed both sides."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import compare, f64, plan, require_gpu, run_fwd
from test_gpu_backward import check, check_lse, output_grad, run_train
from test_gpu_parity import small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def random_case(seed, training=False):
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 4))
    n = int(rng.integers(1, 7))
    S = int(rng.integers(max(n, 2), 420))
    hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4] if training else [1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    rope = str(rng.choice(["none", "1d", "2d", "mrope"]))
    norm = bool(rng.integers(0, 2))
    dtype = "bf16" if training or rng.random() < 0.8 else "f32"
    w = small([W.Segment(W.SEG_CAUSAL, S)], hq=g * hkv, hkv=hkv, d=d, rope=rope, norm=norm,
              batch=batch, dtype=dtype, theta=1e4 if rope == "2d" else 5e6, seed=200 + seed)
    tables = []
    for _ in range(batch):
        cuts = np.sort(rng.choice(np.arange(1, S), size=n - 1, replace=False)) if n > 1 else []
        bounds = [0, *[int(c) for c in cuts], S]
        kinds = rng.integers(0, 4, size=n)
        tables.append([[bounds[s], bounds[s + 1] - bounds[s], int(kinds[s])] for s in range(n)])
    x = dataclasses.replace(W.generate(w), segments=np.array(tables, dtype=np.int32))
    return w, x


@pytest.mark.parametrize("seed", range(24))
def test_forward_random_layout(seed):
    w, x = random_case(seed)
    parts = [0, 0, 2, 3][seed % 4] if w.dtype == "bf16" else 0
    print(f"case seed {seed}: B={w.batch} S={w.seq_len} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"d={w.head_dim} {w.dtype} rope={w.rope} norm={w.qk_norm} split={parts} "
          f"segments={x.segments.tolist()}", flush=True)
    with plan(split_parts=parts):
        out, _ = run_fwd(x)
    compare(f64(out), oracle.hot_path(x), w.dtype, f"seed {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_backward_random_layout(seed):
    w, x = random_case(seed, training=True)
    print(f"case seed {seed}: B={w.batch} S={w.seq_len} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"d={w.head_dim} rope={w.rope} norm={w.qk_norm} segments={x.segments.tolist()}", flush=True)
    dout = output_grad(w, seed=300 + seed)
    got = run_train(x, dout)
    masks = [oracle.explicit_mask(x.segments[b], w.seq_len) for b in range(w.batch)]
    q_rot, k_rot = oracle.prologue(x)
    check_lse(got["lse"], oracle.attention_lse(q_rot, k_rot, masks))
    want = oracle.path_backward(x, dout)
    for t in ("dq", "dk", "dv"):
        check(f"seed {seed} {t}", got[t], want[t])
    if w.qk_norm:
        for t in ("dw_q", "dw_k"):
            check(f"seed {seed} {t}", got[t], want[t])
