"""Pins of the oracle's grouped output projection (zartbot walkthrough,
section 1.2: o_lora_rank 1024 in o_groups 8) against other statements of it."""
import numpy as np
import pytest
import scipy.linalg

from oracle import csa2


def _data(n, G, R, K, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, G * K)), rng.standard_normal((G, R, K))


@pytest.mark.parametrize("n, G, R, K", [(3, 1, 5, 7), (4, 8, 16, 32), (2, 3, 4, 6)])
def test_equals_block_diagonal_matrix(n, G, R, K):
    # the projection is one matrix product with the block-diagonal matrix of the groups' weights
    x, w = _data(n, G, R, K)
    big = scipy.linalg.block_diag(*w)  # [G R, G K]
    np.testing.assert_allclose(csa2.grouped_out_proj(x, w), x @ big.T, rtol=1e-12, atol=1e-12)


def test_brute_force_sums():
    x, w = _data(2, 2, 3, 4, seed=1)
    y = csa2.grouped_out_proj(x, w)
    for t in range(2):
        for g in range(2):
            for r in range(3):
                want = sum(x[t][g * 4 + c] * w[g][r][c] for c in range(4))
                assert abs(y[t][g * 3 + r] - want) < 1e-12


def test_group_isolation():
    # output group g depends only on input slice g: a change to slice 1 moves outputs of group 1 alone
    x, w = _data(3, 4, 5, 6, seed=2)
    y0 = csa2.grouped_out_proj(x, w)
    x2 = x.copy()
    x2[:, 6:12] += 1.0
    dy = csa2.grouped_out_proj(x2, w) - y0
    assert np.all(dy[:, :5] == 0) and np.all(dy[:, 10:] == 0) and np.any(dy[:, 5:10] != 0)


def test_shape_mismatch_raises():
    x, w = _data(2, 2, 3, 4)
    with pytest.raises(ValueError):
        csa2.grouped_out_proj(x[:, :7], w)
