"""The lower bounds the selection kernel carries from one level to the next.

The kernel selects the top m super-blocks (64 slots) by super-block maximum,
then the top m blocks (8 slots) inside them by block maximum, then the top m
entries inside those blocks, and starts each level's radix search at the
previous level's threshold (the m-th largest key): each chosen group holds a
sub-group (or entry) whose key is the group's own, so at least m keys of the
next level reach that threshold.  With a pool, the forced block and its
super-block carry a key above every score, and the pool's top-k (k <= kappa
- 1) over its members' own keys is bounded by the pool's block threshold.
These tests check the claims by brute force on random scores with many ties
and invalid slots (the kernel's order: score descending, then id ascending).
"""
import numpy as np
import pytest

NEG = -np.inf


def top(keys, m):
    """Indices of the m best keys (value desc, index asc) among the valid ones, and the m-th key."""
    order = sorted((i for i in range(len(keys)) if keys[i] > NEG), key=lambda i: (-keys[i], i))
    chosen = order[:m]
    return chosen, (keys[chosen[-1]] if len(chosen) == m else NEG)


def group_max(scores, size):
    return scores.reshape(-1, size).max(axis=1)


@pytest.mark.parametrize("seed", range(40))
def test_flat_levels_bound_each_other(seed):
    rng = np.random.default_rng(seed)
    n_sb = int(rng.integers(4, 24))
    scores = np.round(rng.normal(size=64 * n_sb), int(rng.integers(0, 3)))  # ties
    scores[rng.random(scores.size) < 0.2] = NEG  # invalid slots
    m = int(rng.integers(1, 8 * n_sb))
    sb = group_max(scores, 64)
    chosen_sb, t1 = top(sb, m)
    # each level's candidates in ascending id order, as the kernel lists them
    # (ties then break by position exactly as by id)
    blocks = [8 * s + i for s in sorted(chosen_sb) for i in range(8)]
    bm = group_max(scores, 8)
    chosen_b, t2 = top(bm[blocks], m)
    assert t2 >= t1  # the block level's m-th key is at least the super-block threshold
    entries = [8 * b + i for b in sorted(blocks[c] for c in chosen_b) for i in range(8)]
    _, t3 = top(scores[entries], m)
    assert t3 >= t2
    # and the hierarchical result is the exact top m (the claim the levels rest on)
    exact, _ = top(scores, m)
    got = sorted(entries[c] for c in top(scores[entries], m)[0])
    assert got == sorted(exact)


@pytest.mark.parametrize("seed", range(40))
def test_pool_thresholds_bound_its_top_k(seed):
    rng = np.random.default_rng(100 + seed)
    n_sb = int(rng.integers(6, 24))
    scores = np.round(rng.normal(size=64 * n_sb), 1)
    n_vis = int(rng.integers(1, scores.size + 1))
    scores[n_vis:] = NEG
    kappa = int(rng.integers(2, 4 * n_sb))
    k = int(rng.integers(1, kappa))  # k <= kappa - 1
    fb = (n_vis - 1) // 8  # the newest visible block is forced in
    sb = group_max(scores, 64)
    forced_sb = sb.copy()
    forced_sb[fb // 8] = np.inf
    chosen_sb, t1 = top(forced_sb, kappa)
    blocks = [8 * s + i for s in sorted(chosen_sb) for i in range(8)]
    bm = group_max(scores, 8)
    forced_bm = bm[blocks].copy()
    forced_bm[blocks.index(fb)] = np.inf
    chosen_b, t_pool = top(forced_bm, kappa)
    assert t_pool >= t1
    pool = sorted(blocks[c] for c in chosen_b)
    assert fb in pool
    own = bm[pool]  # the pool members' own keys, the forced block's real maximum included
    _, t_k = top(own, k)
    assert t_k >= t_pool  # the bound the kernel passes to the pool's top-k


def test_pool_threshold_does_not_bound_a_larger_top_k():
    """Why the kernel drops the bound before a flat top-k that follows a pool
    selection with k >= kappa: the pool's threshold for kappa places lies
    above the k-th largest key."""
    scores = np.repeat(np.arange(16, 0, -1, dtype=np.float64), 64)  # super-block s scores 16 - s
    sb = group_max(scores, 64)
    kappa, k = 2, 10
    _, t_pool_sb = top(sb, kappa)
    _, t_flat = top(sb, k)
    assert t_flat < t_pool_sb
