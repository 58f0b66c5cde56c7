"""csa2_layer_group_noalloc (the layer-group call with the library's own
scratch, for callers that cannot allocate) against csa2_layer_group with a
caller workspace: two calls in a row on one GPU, the second on a smaller
shape than the first (so its scratch region still holds the first call's
data), each bit-identical to the workspace entry point on the same inputs.
"""
from dataclasses import replace

import pytest

import synth

pytestmark = pytest.mark.gpu


def _noalloc_matches_group(R, B, wl):
    import torch

    name = wl.name
    inp = synth.Inputs(wl)
    print(f"[noalloc] {name}: batch {wl.batch}, context {wl.context}, layers {[p.mode for p in wl.layers]}", flush=True)
    st = R.DeviceStep(wl, inp)
    st.run()  # csa2_layer_group with the caller's workspace
    torch.cuda.synchronize()
    ref = [{k: (None if L[k] is None else L[k].clone()) for k in ("topk", "pool", "out", "lse")} for L in st.layers]
    for L in st.layers:  # poison every output
        L["topk"].fill_(-7)
        L["out"].fill_(float("nan"))
        L["lse"].fill_(float("nan"))
        if L["pool"] is not None:
            L["pool"].fill_(-7)
    torch.cuda.synchronize()
    # the same step through the allocation-free entry point (its compress
    # rewrites the step's new entries with the same bytes)
    B.csa2_layer_group_noalloc(st.dims, st.cache.struct(), st.layer_structs(), st.q_pos, wl.n_q, st.compress_args())
    torch.cuda.synchronize()
    for li, (want, L) in enumerate(zip(ref, st.layers)):
        for k in ("topk", "pool", "out", "lse"):
            if want[k] is not None:
                assert torch.equal(want[k], L[k]), f"{name} layer {li}: {k} differs from csa2_layer_group"
    need = B.csa2_workspace_size(st.dims, st.cache.struct(), B.EP_LAYER_GROUP, wl.n_q)
    print(f"[noalloc] {name}: identical ({need} bytes of scratch)", flush=True)
    return need


def test_noalloc_group_matches_workspace_group_twice_shrinking():
    import torch

    assert torch.cuda.is_available()
    from kv_cache_compression_csa2_amd import binding as B
    from kv_cache_compression_csa2_amd import runner as R

    big = synth.get("group_small")  # Full(pool) + Reindex x2 + Reuse, 2 x 20001
    first = _noalloc_matches_group(R, B, big)
    # the same layers over a shorter context: every buffer of the step smaller
    second = _noalloc_matches_group(R, B, replace(big, name="group_short", prior=9000))
    assert second < first


def test_noalloc_group_replays_in_a_hip_graph():
    """The allocation-free entry point captured in a HIP graph, the use it is
    for: every replay, with eager work and synchronisation between replays,
    gives the eager call's top-k, pool, outputs and LSE bit for bit (its
    launches record no memset and stay on the capturing stream)."""
    import torch

    from kv_cache_compression_csa2_amd import binding as B
    from kv_cache_compression_csa2_amd import runner as R

    wl = synth.get("group_small")
    inp = synth.Inputs(wl)
    st = R.DeviceStep(wl, inp)
    cache, layers, compress = st.cache.struct(), st.layer_structs(), st.compress_args()
    # eager first: also this device's first call, which looks up the scratch address
    B.csa2_layer_group_noalloc(st.dims, cache, layers, st.q_pos, wl.n_q, compress)
    torch.cuda.synchronize()
    ref = [{k: (None if L[k] is None else L[k].clone()) for k in ("topk", "pool", "out", "lse")} for L in st.layers]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.csa2_layer_group_noalloc(st.dims, cache, layers, st.q_pos, wl.n_q, compress)
    for rep in range(3):
        for L in st.layers:  # eager work between replays
            L["topk"].fill_(-7)
            L["out"].zero_()
            L["lse"].zero_()
            if L["pool"] is not None:
                L["pool"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"[noalloc] graph replay {rep}", flush=True)
        for li, (want, L) in enumerate(zip(ref, st.layers)):
            for k in ("topk", "pool", "out", "lse"):
                if want[k] is not None:
                    assert torch.equal(want[k], L[k]), f"replay {rep} layer {li}: {k} differs from the eager call"
