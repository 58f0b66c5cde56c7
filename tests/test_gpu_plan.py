"""GPU parity of a model schedule run group by group: csa2_layer_plan groups
the layers by shared cache and each group runs as one csa2_layer_group call
over its own caches, checked against the oracle (cache bytes, sets, pools,
outputs).  The schedule has two groups of the pages' kinds (zartbot
walkthrough 2.3.3): an encoder group at ratio 2 (Full, then Reuse layers)
and a decoder group at ratio 1 (Full building the pool, Reuse, Reindex over
the pool, Reuse)."""
from dataclasses import replace

import pytest

import synth
from oracle import plan as oplan
from tests import harness

pytestmark = pytest.mark.gpu

RATIOS = [0, 2, 2, 2, 1, 1, 1, 1, 1, 1]
KV, IDX, CAND = [1, 4], [1, 4, 7], 4
NAMES = {0: "full", 1: "reindex", 2: "reuse"}
# per-ratio shapes: a small encoder decode (ratio 2) and a small decoder with a non-trivial pool
BASE = {
    2: replace(synth.get("decode_32k"), name="plan_enc", batch=2, ratio=2, prior=12000, new=2, n_q=2),
    1: replace(synth.get("hsi_small"), name="plan_dec"),
}


def test_plan_groups_match_oracle_and_run_with_parity():
    import torch

    assert torch.cuda.is_available()
    from kv_cache_compression_csa2_amd import model, runner

    mp = model.ModelPlan(RATIOS, KV, IDX, CAND)
    ref = oplan.layer_plan(RATIOS, KV, IDX, CAND)
    assert mp.window_only() == [l for l, p in enumerate(ref) if p.mode == "window"]
    groups = mp.groups()
    assert sorted(groups) == KV
    for g, members in groups.items():
        # the group's layers, modes and sources are the oracle plan's
        layers = [m.layer for m in members]
        assert layers == [l for l, p in enumerate(ref) if p.group == g]
        for m in members:
            p = ref[m.layer]
            assert NAMES[m.mode] == p.mode and m.make_pool == p.make_pool
            assert (members[m.source].layer if m.source >= 0 else -1) == p.source
        wl = replace(BASE[mp.ratio_of(g)], name=f"plan_g{g}",
                     layers=tuple(synth.LayerPlan(NAMES[m.mode], m.source, m.make_pool) for m in members))
        inp = synth.Inputs(wl)
        print(f"[plan] group {g}: ratio {wl.ratio}, layers {[NAMES[m.mode] for m in members]}", flush=True)
        step = runner.DeviceStep(wl, inp)
        step.run()
        torch.cuda.synchronize()
        seqs = list(range(wl.batch))
        caches = harness.oracle_caches(inp, seqs)
        harness.compare_cache_bytes(step, caches, seqs)
        summary = harness.check_step(step, inp, seqs, caches)
        print(f"[plan] group {g}: {summary}", flush=True)
