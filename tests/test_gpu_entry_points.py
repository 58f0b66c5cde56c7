"""GPU parity through the standalone entry points of the C ABI.

csa2_layer_group drives the library's internal launchers; these tests call
the exported csa2_compress, csa2_index_topk and csa2_sparse_attn one by one,
the way a caller that runs its own layer loop would:

* Full: csa2_index_topk with topk_scores and pool_out;
* Reindex: csa2_index_topk over that pool (pool_in), with topk_scores;
* Reuse: csa2_sparse_attn with the cache's indexer K pointer NULL (a Reuse
  layer never reads the indexer K: zartbot walkthrough, 3.2 access table);
* attention with no window buffer (n_swa = 0).

Every output must equal the csa2_layer_group run of the same step bit for
bit, and the returned scores must match the oracle's float64 scores of the
same stored bytes within the float32 error bound derived in
score_error_bound().
"""
from dataclasses import replace

import numpy as np
import pytest

import synth
from tests import harness

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mods():
    import torch

    assert torch.cuda.is_available()
    from kv_cache_compression_csa2_amd import binding as B
    from kv_cache_compression_csa2_amd import runner as R

    return B, R


def score_error_bound(q_idx, head_w, k_rows):
    """Bound on |GPU score - exact score| for each row of k_rows.

    The GPU forms each head's dot product of d_idx exact products (bf16 x bf16,
    or fp16 x the exactly dequantised FP4 value) in float32, takes the ReLU
    (1-Lipschitz, so it never enlarges an error), multiplies by the head
    weight and sums the heads in float32 (plus one addition joining two
    partial sums).  Any sum of n terms whose additions each round with
    relative error at most u is within gamma_n = n u / (1 - n u) of the exact
    sum times the sum of the terms' magnitudes (Higham, Accuracy and Stability
    of Numerical Algorithms, 3.1).  u = 2^-23 covers round-to-nearest and any
    faithful rounding inside the matrix cores.  With n_d = d_idx + 1 terms per
    dot and n_h = 2 Hi + 2 operations in the head sum:
        |err| <= sum_h |w_h| gamma_{n_d} sum_e |q_he K_e|
                 + gamma_{n_h} sum_h |w_h| relu(q_h . K)
    plus, for FP4 caches, the query's conversion to fp16 after scaling by a
    power of two that puts its largest magnitude in [2^14, 2^15): elements
    below fp16's normal range round to 2^-24 of that scale, at most
    2^-38 max|q_h| per element.
    """
    u = 2.0 ** -23
    gamma = lambda n: n * u / (1 - n * u)
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(head_w, dtype=np.float64)
    K = np.asarray(k_rows, dtype=np.float64)
    di = q.shape[1]
    absdot = np.abs(K) @ np.abs(q).T  # [n, Hi]
    relu = np.maximum(K @ q.T, 0.0)
    conv = np.abs(K).sum(axis=1, keepdims=True) * (2.0 ** -38 * np.abs(q).max())
    return gamma(di + 1) * (absdot @ np.abs(w)) + gamma(2 * q.shape[0] + 2) * (relu @ np.abs(w)) + (conv[:, 0] * np.abs(w).sum())


def check_scores(gpu_ids, gpu_scores, cache, q_idx, head_w, what):
    ids = np.asarray(gpu_ids)
    sc = np.asarray(gpu_scores, dtype=np.float64)
    kept = ids >= 0
    assert np.all(np.isneginf(sc[~kept])), f"{what}: padding scores must be -inf"
    rows = cache.idx_rows(ids[kept])
    ref = harness.oc.indexer_scores(q_idx, head_w, rows)
    bound = score_error_bound(q_idx, head_w, rows)
    err = np.abs(sc[kept] - ref)
    worst = np.max(err / np.maximum(bound, 1e-300)) if len(err) else 0.0
    assert np.all(err <= bound), f"{what}: score error {err.max():.3g} exceeds its bound (ratio {worst:.3g})"
    return worst


MODES = (synth.LayerPlan("full", make_pool=True), synth.LayerPlan("reindex", 0), synth.LayerPlan("reuse", 1))
CASES = {
    "hsi_small": synth.get("hsi_small"),
    "fp4_small_modes": replace(synth.get("fp4_small"), name="fp4_small_modes", layers=MODES),
}


@pytest.mark.parametrize("name", list(CASES))
def test_standalone_calls_match_group_and_oracle(mods, name):
    import torch

    B, R = mods
    wl = CASES[name]
    inp = synth.Inputs(wl)
    print(f"[entry] {name}: batch {wl.batch}, context {wl.context}, kv {wl.kv}", flush=True)
    ref = R.DeviceStep(wl, inp)
    ref.run()
    torch.cuda.synchronize()

    st = R.DeviceStep(wl, inp)
    ws = st.workspace()
    cs = st.cache.struct()
    B.csa2_compress(st.dims, cs, st.latent_new, st.first_pos, wl.new, st.pair_logits, st.w_ik)
    L0, L1, L2 = st.layers
    dev = st.q_pos.device
    scores0 = torch.empty((wl.batch, wl.n_q, wl.topk), dtype=torch.float32, device=dev)
    scores1 = torch.empty_like(scores0)
    # Full: top-k, pool and scores
    B.csa2_index_topk(st.dims, cs, L0["q_idx"], L0["head_w"], st.q_pos, wl.n_q, None, L0["topk"], L0["pool"],
                      scores0, ws)
    B.csa2_sparse_attn(st.dims, cs, L0["q"], st.q_pos, wl.n_q, L0["topk"], L0["swa"], L0["swa_first"],
                       L0["swa"].shape[1], L0["out"], L0["lse"], ws)
    # Reindex over the Full layer's pool
    B.csa2_index_topk(st.dims, cs, L1["q_idx"], L1["head_w"], st.q_pos, wl.n_q, L0["pool"], L1["topk"], None,
                      scores1, ws)
    B.csa2_sparse_attn(st.dims, cs, L1["q"], st.q_pos, wl.n_q, L1["topk"], L1["swa"], L1["swa_first"],
                       L1["swa"].shape[1], L1["out"], L1["lse"], ws)
    # Reuse: the indexer K is not passed at all
    cs_noidx = st.cache.struct(with_idx=False)
    assert cs_noidx.idx_k is None and cs_noidx.idx_scale is None
    B.csa2_sparse_attn(st.dims, cs_noidx, L2["q"], st.q_pos, wl.n_q, L1["topk"], L2["swa"], L2["swa_first"],
                       L2["swa"].shape[1], L2["out"], L2["lse"], ws)
    L2["topk"].copy_(L1["topk"])  # what the group's Reuse layer records as its top-k
    torch.cuda.synchronize()

    # bit for bit against the layer-group run (its Reuse layer copied the top-k)
    for li, (a, b) in enumerate(zip(ref.layers, st.layers)):
        assert torch.equal(a["topk"], b["topk"]), f"{name} layer {li}: top-k differs from the group run"
        assert torch.equal(a["out"], b["out"]), f"{name} layer {li}: output differs from the group run"
        assert torch.equal(a["lse"], b["lse"]), f"{name} layer {li}: lse differs from the group run"
    assert torch.equal(ref.layers[0]["pool"], L0["pool"]), f"{name}: pool differs from the group run"

    # against the oracle: cache bytes, sets, pool, outputs (harness), then the scores element-wise
    seqs = list(range(wl.batch))
    caches = harness.oracle_caches(inp, seqs)
    harness.compare_cache_bytes(st, caches, seqs)
    summary = harness.check_step(st, inp, seqs, caches)
    specs = harness.driver.layer_specs(inp, seqs)
    worst = 0.0
    for b in seqs:
        for qi in range(wl.n_q):
            worst = max(worst, check_scores(L0["topk"][b, qi].cpu().numpy(), scores0[b, qi].cpu().numpy(), caches[b],
                                            specs[0].q_idx[b, qi], specs[0].head_w[b, qi], f"{name} Full seq {b}"))
            worst = max(worst, check_scores(L1["topk"][b, qi].cpu().numpy(), scores1[b, qi].cpu().numpy(), caches[b],
                                            specs[1].q_idx[b, qi], specs[1].head_w[b, qi], f"{name} Reindex seq {b}"))
    print(f"[entry] {name}: {summary}; worst score error / bound {worst:.3g}", flush=True)


@pytest.mark.parametrize("name", ["tiny_encoder", "hsi_small", "fp4_small"])
def test_attention_without_window(mods, name):
    """csa2_sparse_attn with n_swa = 0 (no window buffer: swa_kv and
    swa_first_pos NULL) attends over the kept rows alone.  tiny_encoder runs
    the float32 plain kernel, the others the matrix-core kernels."""
    import torch

    B, R = mods
    wl = synth.get(name)
    inp = synth.Inputs(wl)
    print(f"[entry] {name}: attention with n_swa = 0", flush=True)
    st = R.DeviceStep(wl, inp)
    st.run()
    torch.cuda.synchronize()
    L0 = st.layers[0]
    out = torch.full_like(L0["out"], float("nan"))
    lse = torch.full_like(L0["lse"], float("nan"))
    B.csa2_sparse_attn(st.dims, st.cache.struct(), L0["q"], st.q_pos, wl.n_q, L0["topk"], None, None, 0, out, lse,
                       st.workspace())
    torch.cuda.synchronize()
    seqs = list(range(wl.batch))
    caches = harness.oracle_caches(inp, seqs)
    spec = harness.driver.layer_specs(inp, seqs)[0]
    q_pos = wl.q_positions()
    got, got_lse = harness.to64(out), lse.cpu().numpy()
    for b in seqs:
        for qi in range(wl.n_q):
            t = int(q_pos[b, qi])
            top = L0["topk"][b, qi].cpu().numpy()
            rows = harness.oc.gather_rows(caches[b], top, np.zeros((0, wl.d)), 0, t, wl.window)
            assert rows.shape[0] == np.count_nonzero(top >= 0)
            o, _, ls = harness.oc.attention(spec.q[b, qi], t, rows, wl.d_rope, harness.driver.rope_cfg(wl))
            harness.check_outputs(got[b, qi], o, wl, f"{name} seq {b} q {qi} (no window)")
            assert np.allclose(got_lse[b, qi], ls, atol=2e-2 if wl.act == "bf16" else 1e-5), f"{name}: lse"


# One-query decode steps with one new entry per sequence, where the layer
# group's first scan writes the entry itself; per sequence: the usual case,
# the query one position before the entry's (the entry is hidden from it),
# fewer entries than the cache holds (the entry past them), a first position
# past the cache (nothing written), and at ratio 2 a first position that is
# not a whole entry (nothing written).
EDGE_CASES = {
    "decode_edges": replace(synth.get("decode_small"), name="decode_edges", batch=4),
    "fp4_edges": replace(synth.get("fp4_small"), name="fp4_edges", batch=4, prior=6000),
    "r2_edges": replace(synth.get("decode_r2_small"), name="r2_edges", batch=5),
}


def _edge_inputs(st, wl):
    st.q_pos[1] -= 1
    st.cache.n_entries[2] = wl.n_prior_entries - 37
    st.first_pos[3] = wl.capacity * wl.ratio
    if wl.batch > 4:
        st.first_pos[4] += 1


@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_fused_decode_entry_edges(mods, name):
    """The layer group's decode scan that also writes the step's entry gives
    the same top-k, pool, outputs, LSE and cache bytes, bit for bit, as the
    separate csa2_compress, csa2_index_topk and csa2_sparse_attn calls."""
    import torch

    B, R = mods
    wl = EDGE_CASES[name]
    inp = synth.Inputs(wl)
    print(f"[entry] {name}: fused decode entry edges, batch {wl.batch}, kv {wl.kv}", flush=True)
    fused = R.DeviceStep(wl, inp)
    sep = R.DeviceStep(wl, inp)
    _edge_inputs(fused, wl)
    _edge_inputs(sep, wl)
    torch.cuda.synchronize()
    B.csa2_trace_enable(64)
    try:
        fused.run()
        torch.cuda.synchronize()
        recs, _ = B.csa2_trace_read()
    finally:
        B.csa2_trace_enable(0)
    names = [n for n, _ in recs]
    assert names[0].startswith("scan_fused_") and "compress_kernel" not in names, names

    cs, ws = sep.cache.struct(), sep.workspace()
    B.csa2_compress(sep.dims, cs, sep.latent_new, sep.first_pos, wl.new, sep.pair_logits, sep.w_ik)
    L = sep.layers[0]
    B.csa2_index_topk(sep.dims, cs, L["q_idx"], L["head_w"], sep.q_pos, wl.n_q, None, L["topk"], L["pool"], None, ws)
    B.csa2_sparse_attn(sep.dims, cs, L["q"], sep.q_pos, wl.n_q, L["topk"], L["swa"], L["swa_first"],
                       L["swa"].shape[1], L["out"], L["lse"], ws)
    torch.cuda.synchronize()

    F = fused.layers[0]
    for key in ("topk", "out", "lse") + (("pool",) if L["pool"] is not None else ()):
        assert torch.equal(F[key], L[key]), f"{name}: {key} differs between the fused and the separate calls"
    for attr in ("main", "main_scale", "idx_store", "idx_scale"):
        a, b = getattr(fused.cache, attr), getattr(sep.cache, attr)
        assert (a is None) == (b is None) and (a is None or torch.equal(a, b)), f"{name}: cache {attr} differs"
    # where the new entry is hidden from the query or past the entries, the top-k leaves it out
    j = wl.n_prior_entries
    top = F["topk"].cpu().numpy()
    for b in (1, 2):
        assert not (top[b] == j).any(), f"{name}: seq {b} keeps entry {j}"
    if wl.batch > 4:  # no entry written at an odd position: the cache row stays as the prior build left it
        assert not fused.cache.main[4, j].any() and not sep.cache.main[4, j].any(), f"{name}: seq 4 wrote entry {j}"
