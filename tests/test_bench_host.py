"""The benchmark's useful-work count, on the CPU.

bench.py reports useful attention FLOPs as 4 * d * Hq per allowed query-key pair, with the
pairs counted in closed form from the segment table. Here that count is held to the
golden pair counts of every workload (sums of the explicit mask, written by the oracle) and
to the oracle's explicit mask on seeded random layouts of every segment kind, so that the
numerator of the reported metric cannot drift from the mask the path computes (HiDream-O1
model card, "What this model is": causal text, full image rows; HunyuanImage 3.0 digest,
"Generalized Causal Attention" and the multi-image training mask).
"""
import json
import os

import numpy as np
import pytest

import bench
import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_allowed_pairs_match_golden_counts():
    gold = json.load(open(os.path.join(GOLDEN, "pair_counts.json")))["counts"]
    for name, entry in gold.items():
        w = W.CONFIGS[name]
        table = W.segment_table(w)
        for b in range(w.batch):
            assert bench.allowed_pairs(table[b], w.seq_len) == entry["allowed_pairs_per_batch_item"], (name, b)


def test_allowed_pairs_match_explicit_mask_on_random_layouts():
    rng = np.random.default_rng(20261204)
    for case in range(40):
        n_seg = int(rng.integers(1, 7))
        lengths = rng.integers(1, 40, size=n_seg)
        kinds = rng.integers(0, 4, size=n_seg)
        starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
        table = np.stack([starts, lengths, kinds], axis=1).astype(np.int64)
        S = int(lengths.sum())
        want = int(oracle.mask.explicit_mask(table, S).sum())
        assert bench.allowed_pairs(table, S) == want, (case, table.tolist())


@pytest.mark.parametrize("name", ["hd2048", "edit", "hunyuan", "hunyuan_multigen"])
def test_pairs_of_the_whole_batch(name):
    """The batch total the metric uses: every item of these workloads has the same layout."""
    gold = json.load(open(os.path.join(GOLDEN, "pair_counts.json")))["counts"][name]
    w = W.CONFIGS[name]
    table = W.segment_table(w)
    pairs = sum(bench.allowed_pairs(table[b], w.seq_len) for b in range(w.batch))
    assert pairs == w.batch * gold["allowed_pairs_per_batch_item"]


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    """One GPU only: more exits with status 2 and says so, before anything touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
