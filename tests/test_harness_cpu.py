"""The parity comparisons themselves, on the CPU: each accepts the oracle's own
answer and the differences its rules allow, and rejects a planted mistake
(a wrong entry, a missing forced block, an output off by more than the bar),
so a lenient comparison cannot hide a wrong GPU result.
"""
import numpy as np
import pytest

from oracle import csa2 as oc
from tests import harness


def _domain(n=200, seed=0):
    rng = np.random.default_rng(seed)
    ids = np.arange(n)
    scores = rng.standard_normal(n)
    return ids, scores


def _oracle_topk(ids, scores, k):
    order = oc.rank_order(scores, ids)
    return np.sort(ids[order[:k]]), order


def test_index_set_accepts_the_oracle_and_rejects_a_wrong_entry():
    ids, scores = _domain()
    k = 32
    ref, order = _oracle_topk(ids, scores, k)
    assert harness.check_index_set(np.concatenate([ref, [-1] * 8]), ids, scores, k) == 0
    # swap the k-th entry for one far below the threshold: the gap is not a tie
    wrong = ref.copy()
    wrong[wrong == ids[order[k - 1]]] = ids[order[-1]]
    with pytest.raises(AssertionError):
        harness.check_index_set(np.sort(wrong), ids, scores, k)


def test_index_set_allows_swaps_inside_the_tie_band_only():
    ids, scores = _domain()
    k = 32
    ref, order = _oracle_topk(ids, scores, k)
    kth, nxt = ids[order[k - 1]], ids[order[k]]
    tied = scores.copy()
    tied[nxt] = tied[kth] * (1 - 1e-5)  # within 1e-3 of the k-th score
    ref, order = _oracle_topk(ids, tied, k)
    swapped = ref.copy()
    swapped[swapped == kth] = nxt
    assert harness.check_index_set(np.sort(swapped), ids, tied, k) == 2
    # the same swap with a real gap fails
    gapped = scores.copy()
    gapped[nxt] = gapped[kth] - 0.5 * abs(gapped[kth]) - 0.1
    with pytest.raises(AssertionError):
        harness.check_index_set(np.sort(swapped), ids, gapped, k)


def test_index_set_rejects_bad_order_padding_and_count():
    ids, scores = _domain()
    k = 16
    ref, _ = _oracle_topk(ids, scores, k)
    with pytest.raises(AssertionError):  # not ascending
        harness.check_index_set(ref[::-1], ids, scores, k)
    with pytest.raises(AssertionError):  # a duplicate
        harness.check_index_set(np.sort(np.concatenate([ref[:-1], ref[:1]])), ids, scores, k)
    with pytest.raises(AssertionError):  # padding other than -1
        harness.check_index_set(np.concatenate([ref, [-2]]), ids, scores, k)
    with pytest.raises(AssertionError):  # one entry short
        harness.check_index_set(np.concatenate([ref[:-1], [-1]]), ids, scores, k)


def test_index_set_small_domain_must_be_kept_whole():
    ids, scores = _domain(n=10)
    assert harness.check_index_set(np.concatenate([ids, [-1] * 6]), ids, scores, 16) == 0
    with pytest.raises(AssertionError):
        harness.check_index_set(np.concatenate([ids[:-1], [-1] * 7]), ids, scores, 16)


def test_pool_accepts_the_oracle_and_rejects_a_missing_forced_block():
    rng = np.random.default_rng(1)
    beta, kappa = 8, 16
    scores = rng.standard_normal(8 * 64 + 3)  # 65 blocks, the last one partial
    nb = -(-len(scores) // beta)
    forced = (len(scores) - 1) // beta
    bmax = oc.block_maxima(scores, beta)
    others = np.array([b for b in range(nb) if b != forced])
    best = others[oc.rank_order(bmax[others], others)[: kappa - 1]]
    pool = np.sort(np.concatenate([best, [forced]]))
    harness.check_pool(pool, scores, beta, kappa)
    # the forced block replaced by the next-best other block
    nxt = others[oc.rank_order(bmax[others], others)[kappa - 1]]
    with pytest.raises(AssertionError):
        harness.check_pool(np.sort(np.concatenate([best, [nxt]])), scores, beta, kappa)
    # a pool that should hold every block
    few = scores[: 8 * 10]
    harness.check_pool(np.array(list(range(10)) + [-1] * (kappa - 10)), few, beta, kappa)
    with pytest.raises(AssertionError):
        harness.check_pool(np.array(list(range(9)) + [-1] * (kappa - 9)), few, beta, kappa)


class _Wl:
    def __init__(self, act):
        self.act = act


def test_outputs_bar():
    rng = np.random.default_rng(2)
    ref = rng.standard_normal((4, 64))
    wl = _Wl("bf16")
    harness.check_outputs(ref + 1e-3 * rng.standard_normal(ref.shape), ref, wl)
    bad = ref.copy()
    bad[1, 7] += 3e-2  # one element past the 2e-2 max-abs bar
    with pytest.raises(AssertionError):
        harness.check_outputs(bad, ref, wl)
    with pytest.raises(AssertionError):  # float32 bar
        harness.check_outputs(ref + 1e-3, ref, _Wl("f32"))
