"""Host-side logic of the torch layer that runs without a GPU."""
import numpy as np
import pytest

import oracle
from unified_text_pixel_amd.api import prefix_is_invariant


def _brute(table, S, p):
    """Rows < p x keys >= p of the explicit mask empty in every item."""
    return all(not oracle.explicit_mask(item, S)[:p, p:].any() for item in table)


def _random_table(rng, batch, S):
    items = []
    for _ in range(batch):
        cuts = np.sort(rng.choice(np.arange(1, S), size=min(S - 1, int(rng.integers(0, 5))), replace=False))
        bounds = [0, *cuts.tolist(), S]
        items.append([[a, b - a, int(rng.integers(0, 4))] for a, b in zip(bounds, bounds[1:])])
    n = max(len(it) for it in items)
    for it in items:
        it += [[S, 0, 0]] * (n - len(it))
    return np.array(items, dtype=np.int32)


@pytest.mark.parametrize("seed", range(40))
def test_prefix_is_invariant_matches_the_mask(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(2, 40))
    table = _random_table(rng, int(rng.integers(1, 4)), S)
    for p in range(S + 1):
        assert prefix_is_invariant(table, S, p) == _brute(table, S, p), (p, table.tolist())


def test_prefix_is_invariant_page_layouts():
    hd = [[[0, 258, 0], [258, 4096, 1]]] * 2
    assert prefix_is_invariant(hd, 4354, 258)          # the text end
    assert prefix_is_invariant(hd, 4354, 100)          # inside the text
    assert not prefix_is_invariant(hd, 4354, 259)      # inside the generation grid
    assert not prefix_is_invariant(hd, 4354, -1) and not prefix_is_invariant(hd, 4354, 4355)
    gca = [[[0, 33, 0], [33, 64, 2], [97, 17, 0]]]
    assert prefix_is_invariant(gca, 114, 33) and prefix_is_invariant(gca, 114, 97)
    assert not prefix_is_invariant(gca, 114, 50)       # splits an image
