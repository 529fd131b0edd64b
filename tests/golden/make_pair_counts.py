"""Write pair_counts.json and tile_counts.json from the oracle alone.

Run from the repository root:  python tests/golden/make_pair_counts.py
Calls only `oracle` (and the input-layout tables in `workloads`).
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    pairs, tiles, tiles_end = {}, {}, {}
    for name, w in workloads.CONFIGS.items():
        table = workloads.segment_table(w)[0]
        M = oracle.explicit_mask(table, w.seq_len)
        pairs[name] = {"seq_len": w.seq_len, "allowed_pairs_per_batch_item": int(M.sum()),
                       "batch": w.batch}
        lab = oracle.tile_labels(M, 64, 64)
        tiles[name] = {"block_q": 64, "block_k": 64,
                       "skip": int((lab == 0).sum()), "full": int((lab == 1).sum()),
                       "partial": int((lab == 2).sum())}
        lab = oracle.tile_labels(M, 64, 64, q_end_aligned=True)
        tiles_end[name] = {"block_q": 64, "block_k": 64,
                           "skip": int((lab == 0).sum()), "full": int((lab == 1).sum()),
                           "partial": int((lab == 2).sum())}
    with open(os.path.join(HERE, "pair_counts.json"), "w") as f:
        json.dump({"source": "oracle.explicit_mask over workloads.CONFIGS (mask rules: HiDream-O1 "
                             "atlas 'How it works'; HunyuanImage 3.0 digest 'Generalized Causal "
                             "Attention')", "counts": pairs}, f, indent=1, sort_keys=True)
    with open(os.path.join(HERE, "tile_counts.json"), "w") as f:
        json.dump({"source": "oracle.tile_labels(oracle.explicit_mask(...), 64, 64), query "
                             "blocks from index 0 (counts) and end-aligned "
                             "(counts_q_end_aligned)",
                   "counts": tiles, "counts_q_end_aligned": tiles_end}, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
