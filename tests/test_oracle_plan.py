"""The cross-layer plan: the oracle's plan pinned to the pages' block
structure and footprint, and the library's csa2_layer_plan (host logic,
callable without a GPU) checked against it."""
import itertools

import numpy as np
import pytest

from oracle import formats, plan

from kv_cache_compression_csa2_amd import binding as B

MODE = {B.FULL: "full", B.REINDEX: "reindex", B.REUSE: "reuse", -1: "window"}


def _pages_plan():
    return plan.layer_plan(plan.PAGES_RATIOS, plan.PAGES_KV_SOURCES, plan.PAGES_INDEX_SOURCES,
                           plan.PAGES_CANDIDATE_SOURCE)


def test_pages_plan_is_the_described_block_structure():
    """zartbot walkthrough 2.3.3 and 3.3.3, written out by hand: layers 0-1
    keep no compressed KV; three encoder blocks of one Full layer and five
    Reuse layers (2-7, 8-13, 14-19); the decoder's Full layer 20 builds the
    pool, Reindex layers 24, 28, 32, 36 search it, and every other decoder
    layer reuses the most recent index layer."""
    p = _pages_plan()
    assert [x.mode for x in p[:2]] == ["window", "window"]
    for head in (2, 8, 14):
        assert p[head] == plan.PlannedLayer(head, "full", -1, False)
        for l in range(head + 1, head + 6):
            assert p[l] == plan.PlannedLayer(head, "reuse", head), l
    assert p[20] == plan.PlannedLayer(20, "full", -1, True)
    for head in (24, 28, 32, 36):
        assert p[head] == plan.PlannedLayer(20, "reindex", 20), head
    for l in range(21, 40):
        if l not in (24, 28, 32, 36):
            latest = max(h for h in (20, 24, 28, 32, 36) if h < l)
            assert p[l] == plan.PlannedLayer(20, "reuse", latest), l
    # counts the pages give: 3 x (1 Full + 5 Reuse) in the encoder, 1 Full + 4 Reindex in the decoder
    assert sum(x.mode == "full" for x in p) == 4 and sum(x.mode == "reindex" for x in p) == 4
    assert sum(x.mode == "reuse" for x in p) == 15 + 15


def test_pages_plan_stores_890_bytes_per_token():
    """The plan's caches in the pages' FP4 format (main KV 288 B, indexer K 68
    B: zartbot walkthrough 3.1) hold 890 B per token, the figure the pages
    print: three ratio-2 encoder groups and one ratio-1 decoder group."""
    main_b = formats.fp4_entry_bytes(512, 16)
    idx_b = formats.fp4_entry_bytes(128, 32)
    assert (main_b, idx_b) == (288, 68)
    assert plan.cache_bytes_per_token(_pages_plan(), plan.PAGES_RATIOS, main_b, idx_b) == 890


def test_plan_rejects_inconsistent_schedules():
    with pytest.raises(ValueError):
        plan.layer_plan((1, 1, 2), (0,), (0,), -1)  # a group mixing ratios
    with pytest.raises(ValueError):
        plan.layer_plan((1, 1), (0,), (1,), -1)  # kv source that is not an index source
    with pytest.raises(ValueError):
        plan.layer_plan((0, 1, 1), (2,), (2,), -1)  # layer 1 has compressed KV before any source


def _library_plan(ratios, kv, idx, cand):
    return [plan.PlannedLayer(g, MODE[m], s, bool(mp)) for g, m, s, mp in B.csa2_layer_plan(ratios, kv, idx, cand)]


def test_library_plan_equals_oracle_on_the_pages_schedule():
    assert _library_plan(plan.PAGES_RATIOS, plan.PAGES_KV_SOURCES, plan.PAGES_INDEX_SOURCES,
                         plan.PAGES_CANDIDATE_SOURCE) == _pages_plan()


def test_library_plan_equals_oracle_on_random_schedules():
    rng = np.random.default_rng(11)
    checked = 0
    for trial in range(400):
        n = int(rng.integers(1, 24))
        # segments of one ratio, each opened by a kv source; a few window-only layers up front
        lead = int(rng.integers(0, 3))
        ratios, kv, idx = [0] * min(lead, n), [], []
        while len(ratios) < n:
            r = int(rng.integers(1, 3))
            seg = int(rng.integers(1, 8))
            start = len(ratios)
            kv.append(start)
            idx.append(start)
            for l in range(start + 1, min(n, start + seg)):
                if rng.random() < 0.3:
                    idx.append(l)
            ratios += [r] * min(seg, n - start)
        cand = int(rng.choice(kv)) if kv and rng.random() < 0.7 else -1
        assert _library_plan(ratios, kv, idx, cand) == plan.layer_plan(ratios, kv, idx, cand), (ratios, kv, idx, cand)
        checked += 1
    assert checked == 400


@pytest.mark.parametrize(
    "ratios,kv,idx,cand",
    [
        ((1, 1, 2), (0,), (0,), -1),       # a group mixing ratios
        ((1, 1), (0,), (1,), -1),          # kv source that is not an index source
        ((0, 1, 1), (2,), (2,), -1),       # compressed KV before any source
        ((1, 1), (1, 0), (0, 1), -1),      # unsorted list
        ((1, 1), (0,), (0,), 1),           # candidate source that is not a kv source
        ((0, 1), (0,), (0,), -1),          # kv source with ratio 0
        ((3, 1), (0,), (0,), -1),          # ratio 3
    ],
)
def test_library_plan_rejects_inconsistent_schedules(ratios, kv, idx, cand):
    with pytest.raises(B.Csa2Error):
        B.csa2_layer_plan(list(ratios), list(kv), list(idx), cand)


def test_decoder_group_workload_is_the_plan_of_layer_20():
    """The decoder group the bounded-replay workloads run is the oracle plan's
    group of layer 20 (modes and sources as positions in the group)."""
    import synth

    p = _pages_plan()
    members = [l for l, x in enumerate(p) if x.group == 20]
    want = [(p[l].mode, members.index(p[l].source) if p[l].source >= 0 else -1, p[l].make_pool) for l in members]
    assert [(x.mode, x.source, x.make_pool) for x in synth.DECODER_GROUP] == want


def test_replay_window_is_the_replayed_segment():
    """Bounded replay (zartbot walkthrough 2.2.2): the window buffer holds only
    the 128 replayed positions, so the segment's first query sees one window
    row (itself) and its last sees all 128."""
    import numpy as np

    import synth
    from oracle import csa2

    wl = synth.get("replay_64k")
    first, n = wl.swa_span()
    q = wl.q_positions()[0]
    assert (first, n) == (65536 - 128, 128) and q[0] == first and q[-1] == 65535
    swa = np.zeros((n, 4))
    cache = csa2.SeqCache("f32", 32, 32, {"f32": np.zeros((1, 4), np.float32)}, {"f32": np.zeros((1, 4), np.float32)})
    rows = [len(csa2.gather_rows(cache, np.array([-1]), swa, first, int(t), wl.window)) for t in (q[0], q[63], q[-1])]
    assert rows == [1, 64, 128]
