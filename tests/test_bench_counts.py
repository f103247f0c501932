"""The flop counts bench.py reports, checked by brute force on small sequences."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _pairs_brute(n, causal):
    qb, kb = -(-n // 128), -(-n // 64)
    out = np.zeros((qb, kb))
    for r in range(n):
        for c in range(n):
            if not causal or c <= r:
                out[r // 128, c // 64] += 1
    return out


@pytest.mark.parametrize("n", [1, 63, 64, 129, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_tile_pairs(n, causal):
    assert np.array_equal(bench.tile_pairs(n, causal), _pairs_brute(n, causal))


def test_effective_flops():
    rng = np.random.default_rng(0)
    n, d = 700, 64
    mask = (rng.random((2, 3, 6, 11)) < 0.4).astype(np.uint8)
    for causal in (False, True):
        pairs = _pairs_brute(n, causal)
        want = 4.0 * d * float((mask * pairs[None, None]).sum())
        assert bench.effective_flops(mask, n, d, causal) == want
    dense = np.ones((1, 1, 6, 11), dtype=np.uint8)
    assert bench.effective_flops(dense, n, d) == 4.0 * d * n * n
    assert bench.effective_flops(dense, n, d, True) == 4.0 * d * n * (n + 1) / 2
