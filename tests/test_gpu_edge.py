"""GPU parity on the degenerate cases of the method, through the C ABI.

Each case runs a whole step (compress, index, select, attend) on small
seeded inputs altered at the source, so the HIP path and the float64 oracle
see the same altered tensors:

* every indexer score equal (zero indexer queries): the top-k and the HSI
  pool are then fixed by the tie rule alone (lower ids first), checked
  exactly;
* every head weight negative: all scores are <= 0, so the selection runs on
  the negative half of the order-preserving keys;
* a sequence with no visible entry: top-k and pool all -1, attention over the
  window rows alone;
* a window buffer that holds only the newest rows: the older window
  positions are skipped;
* the largest top-k and pool the boundary accepts (2048 entries, 2048
  blocks), with the HSI pool built from more blocks than it keeps;
* a context of four entries (less than one HSI block).
"""
from dataclasses import replace

import numpy as np
import pytest

import synth
from synth import LayerPlan
from tests import harness

pytestmark = pytest.mark.gpu


class ZeroIndexQuery(synth.Inputs):
    def q_idx(self, layer):
        return np.zeros_like(super().q_idx(layer))


class NegativeHeadWeights(synth.Inputs):
    def head_w(self, layer):
        return -np.abs(super().head_w(layer))


class TruncatedWindow(synth.Inputs):
    KEEP = 50

    def swa(self, layer):
        rows, first = super().swa(layer)
        drop = rows.shape[1] - self.KEEP
        return np.ascontiguousarray(rows[:, drop:]), first + drop


class _NoEntries:
    """An oracle cache seen with no entries (the GPU sequence gets n_entries = 0)."""

    n_entries = 0

    def __init__(self, cache):
        self._cache = cache

    def __getattr__(self, name):
        return getattr(self._cache, name)


HSI = (LayerPlan("full", make_pool=True), LayerPlan("reindex", 0), LayerPlan("reuse", 1))


def _run(wl, inp, empty_seq=None):
    import torch

    from kv_cache_compression_csa2_amd import runner

    print(f"[edge] {wl.name}: batch {wl.batch}, context {wl.context}, topk {wl.topk}, "
          f"cand {wl.cand_blocks}, inputs {type(inp).__name__}", flush=True)
    step = runner.DeviceStep(wl, inp)
    if empty_seq is not None:
        step.cache.n_entries[empty_seq] = 0
    step.run()
    torch.cuda.synchronize()
    seqs = list(range(wl.batch))
    caches = harness.oracle_caches(inp, seqs)
    harness.compare_cache_bytes(step, caches, seqs)
    if empty_seq is not None:
        caches[empty_seq] = _NoEntries(caches[empty_seq])
    summary = harness.check_step(step, inp, seqs, caches)
    print(f"[edge] {wl.name}: {summary}", flush=True)
    return step


def test_all_scores_tied():
    wl = replace(synth.get("hsi_small"), name="edge_ties")
    step = _run(wl, ZeroIndexQuery(wl))
    k, kappa = wl.topk, wl.cand_blocks
    n_vis = wl.capacity  # the query sits at the last position: every entry is visible
    nb = (n_vis + 7) // 8
    forced = (n_vis - 1) // 8
    pool = step.layers[0]["pool"].cpu().numpy()
    want_pool = np.array(sorted(set(range(kappa - 1)) | {forced}) if nb > kappa else list(range(nb)))
    for b in range(wl.batch):
        # Full: the k lowest ids; pool: the forced block plus the lowest others
        assert np.array_equal(step.layers[0]["topk"].cpu().numpy()[b, 0], np.arange(k))
        assert np.array_equal(pool[b, 0][: len(want_pool)], want_pool)
        # Reindex over that pool: the k lowest ids of the pool's entries
        dom = np.concatenate([np.arange(8 * blk, min(8 * blk + 8, n_vis)) for blk in want_pool])
        assert np.array_equal(step.layers[1]["topk"].cpu().numpy()[b, 0], np.sort(dom)[:k])


def test_negative_scores():
    wl = replace(synth.get("decode_small"), name="edge_negative")
    _run(wl, NegativeHeadWeights(wl))


def test_sequence_without_entries():
    wl = replace(synth.get("hsi_small"), name="edge_empty")
    step = _run(wl, synth.Inputs(wl), empty_seq=1)
    for L in step.layers:
        assert np.all(L["topk"].cpu().numpy()[1] == -1)
    assert np.all(step.layers[0]["pool"].cpu().numpy()[1] == -1)
    assert np.all(np.isfinite(step.layers[0]["out"].float().cpu().numpy()[1]))


def test_window_buffer_holds_newest_rows_only():
    wl = replace(synth.get("multi_q_small"), name="edge_window")
    _run(wl, TruncatedWindow(wl))


def test_largest_topk_and_pool():
    wl = replace(synth.get("decode_32k"), name="edge_max", batch=2, prior=40000, new=1, topk=2048,
                 cand_blocks=2048, layers=HSI)
    _run(wl, synth.Inputs(wl))


def test_context_shorter_than_a_block():
    wl = replace(synth.get("decode_32k"), name="edge_short", batch=2, prior=3, new=1, layers=HSI)
    _run(wl, synth.Inputs(wl))
