"""The library's host-side token permutations against the oracle's (no GPU needed)."""
import ctypes

import numpy as np
import pytest

import block_sparse_attention_sparge_amd as sp
import oracle

GRIDS = [(0, 2, 3, 5), (226, 13, 30, 45), (256, 5, 9, 16), (0, 21, 45, 80), (3, 1, 1, 1), (7, 6, 4, 9)]


@pytest.mark.parametrize("n_text,T,H,W", GRIDS)
def test_cube_permutation_matches_oracle(n_text, T, H, W):
    got = sp.token_permutation(n_text, (T, H, W), "cube").numpy()
    assert np.array_equal(got, oracle.cube_permutation(n_text, T, H, W, (4, 4, 4)))
    got = sp.token_permutation(n_text, (T, H, W), "cube", cube=(2, 3, 5)).numpy()
    assert np.array_equal(got, oracle.cube_permutation(n_text, T, H, W, (2, 3, 5)))


@pytest.mark.parametrize("n_text,T,H,W", GRIDS)
def test_morton_permutation_matches_oracle(n_text, T, H, W):
    got = sp.token_permutation(n_text, (T, H, W), "morton").numpy()
    assert np.array_equal(got, oracle.morton_permutation(n_text, T, H, W))


def test_raster_is_identity_and_errors():
    assert np.array_equal(sp.token_permutation(5, (2, 3, 4), "raster").numpy(), np.arange(29))
    lib = sp.load_library()
    buf = (ctypes.c_int32 * 64)()
    c3 = (ctypes.c_int64 * 3)(4, 4, 4)
    bad_cube = (ctypes.c_int64 * 3)(4, 0, 4)
    assert lib.sparge_token_permutation(0, 2, 2, 2, 1, c3, None) == -1          # NULL
    assert lib.sparge_token_permutation(-1, 2, 2, 2, 1, c3, buf) == -7          # ARG
    assert lib.sparge_token_permutation(0, 0, 2, 2, 1, c3, buf) == -7
    assert lib.sparge_token_permutation(0, 2, 2, 2, 9, c3, buf) == -7
    assert lib.sparge_token_permutation(0, 2, 2, 2, 1, bad_cube, buf) == -7
    assert lib.sparge_token_permutation(0, 2, 2, 2, 1, None, buf) == -7
    assert lib.sparge_token_permutation(0, 1 << 16, 1 << 16, 1 << 16, 0, c3, buf) == -7   # > 2^31 tokens
    with pytest.raises(ValueError):
        sp.token_permutation(0, (2, 2, 2), "spiral")
