"""Helpers for GPU-vs-oracle parity: run both sides on the same seeded inputs and compare.

Comparison rules:
* index sets: equal, unless the oracle's k-th and (k+1)-th scores lie within
  a relative 1e-3 of each other; then only entries whose oracle score is
  within 1e-3 (relative) of the k-th score may differ.  The same rule
  applies to HSI pool blocks at the kappa boundary (on block maxima).
* attention outputs are compared given the GPU's own index set: bf16 / FP4
  max-abs <= 2e-2 and relative L2 <= 5e-3; float32 max-abs <= 1e-4 and
  relative L2 <= 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import csa2 as oc
from oracle import driver

REL_BAND = 1e-3
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-4, 1e-5)}


def tol_for(wl):
    return TOL["f32"] if wl.act == "f32" else TOL["bf16"]


def check_index_set(gpu_ids, dom_ids, dom_scores, k, what=""):
    """GPU top-k list vs the oracle's ranking of a domain (ids + float64 scores)."""
    gpu_ids = np.asarray(gpu_ids)
    kept = gpu_ids[gpu_ids >= 0]
    assert np.all(np.diff(kept) > 0), f"{what}: ids not ascending/unique"
    assert np.all(gpu_ids[len(kept):] == -1), f"{what}: padding not -1"
    dom_ids = np.asarray(dom_ids)
    n = len(dom_ids)
    assert len(kept) == min(k, n), f"{what}: kept {len(kept)} of {n}, k={k}"
    if n <= k:
        assert set(kept.tolist()) == set(dom_ids.tolist()), f"{what}: domain not fully kept"
        return 0
    order = oc.rank_order(dom_scores, dom_ids)
    sk, sk1 = dom_scores[order[k - 1]], dom_scores[order[k]]
    ref = set(dom_ids[order[:k]].tolist())
    got = set(kept.tolist())
    if ref == got:
        return 0
    scale = max(abs(sk), 1e-6 * np.max(np.abs(dom_scores)))
    gap = (sk - sk1) / scale
    assert gap <= REL_BAND, f"{what}: sets differ although the boundary gap is {gap:.3g}"
    by_id = dict(zip(dom_ids.tolist(), dom_scores.tolist()))
    for j in ref ^ got:
        assert abs(by_id[j] - sk) <= REL_BAND * scale, f"{what}: entry {j} differs outside the tie band"
    return len(ref ^ got)


def check_pool(gpu_pool, scores, beta, kappa, what=""):
    """GPU HSI pool vs the oracle's block maxima of the full scores (visible prefix)."""
    gpu_pool = np.asarray(gpu_pool)
    n_vis = len(scores)
    nb = -(-n_vis // beta)
    if nb <= kappa:
        assert list(gpu_pool) == list(range(nb)) + [-1] * (kappa - nb), f"{what}: pool should hold every block"
        return
    forced = (n_vis - 1) // beta
    assert forced in set(gpu_pool.tolist()), f"{what}: forced block missing"
    bmax = oc.block_maxima(scores, beta)
    others = np.array([b for b in range(nb) if b != forced])
    got_others = np.array([b for b in gpu_pool if b != forced and b >= 0])
    check_index_set(got_others, others, bmax[others], kappa - 1, what + " pool")


def oracle_caches(inp, seqs):
    """Oracle caches after the step (prior + new entries) for sequences seqs."""
    wl = inp.wl
    out = []
    for b in seqs:
        c = driver.build_cache(inp, b, wl.context)
        out.append(c)
    return out


def compare_cache_bytes(step, caches, seqs):
    """GPU-written cache rows vs the oracle's stored bytes: exact."""
    wl = step.wl
    n = wl.capacity
    for i, b in enumerate(seqs):
        c = caches[i]
        if wl.kv == "fp4":
            pairs = [(step.cache.main[b, :n], c.main_raw["codes"]), (step.cache.main_scale[b, :n], c.main_raw["scales"]),
                     (step.cache.idx[b, :n], c.idx_raw["codes"]), (step.cache.idx_scale[b, :n], c.idx_raw["scales"])]
            for got, ref in pairs:
                g = got.cpu().numpy()
                bad = np.count_nonzero(g != ref)
                assert bad == 0, f"seq {b}: {bad} FP4 bytes differ"
        else:
            key = "bf16" if wl.kv == "bf16" else "f32"
            for got, ref in ((step.cache.main[b, :n], c.main_raw[key]), (step.cache.idx[b, :n], c.idx_raw[key])):
                g = got.cpu()
                g = g.view(torch.int16).numpy().view(np.uint16) if key == "bf16" else g.numpy()
                bad = np.count_nonzero(g != ref)
                assert bad == 0, f"seq {b}: {bad} {key} elements differ"


def to64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_outputs(got, ref, wl, what=""):
    max_abs, rel = tol_for(wl)
    err = np.max(np.abs(got - ref))
    rl2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= max_abs and rl2 <= rel, f"{what}: max-abs {err:.3g} (<= {max_abs}), rel-L2 {rl2:.3g} (<= {rel})"
    return err, rl2


def check_step(step, inp, seqs=None, caches=None, queries=None):
    """Full parity of one executed GPU step against the oracle on sequences seqs
    (and query indices `queries`, default all).

    Returns a summary dict (counts of tie-band differences, worst errors).
    """
    wl = inp.wl
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    dims = driver.dims_of(wl)
    caches = caches if caches is not None else oracle_caches(inp, seqs)
    specs = driver.layer_specs(inp, seqs)
    q_pos = wl.q_positions()
    summary = {"tie_diffs": 0, "max_abs": 0.0, "rel_l2": 0.0}
    gpu_topk = [L["topk"].cpu().numpy() for L in step.layers]
    gpu_pool = [None if L["pool"] is None else L["pool"].cpu().numpy() for L in step.layers]
    for li, (L, spec) in enumerate(zip(step.layers, specs)):
        plan = L["plan"]
        out = to64(L["out"])
        lse = L["lse"].cpu().numpy()
        for i, b in enumerate(seqs):
            cache = caches[i]
            for qi in (range(wl.n_q) if queries is None else queries):
                t = int(q_pos[b, qi])
                tag = f"{wl.name} layer {li} ({plan.mode}) seq {b} q {qi}"
                n_vis = oc.visible_entries(cache.n_entries, t, wl.ratio)
                top = gpu_topk[li][b, qi]
                if plan.mode == "full":
                    s = oc.full_scores(cache, n_vis, spec.q_idx[i, qi], spec.head_w[i, qi])
                    summary["tie_diffs"] += check_index_set(top, np.arange(n_vis), s, wl.topk, tag)
                    if plan.make_pool:
                        check_pool(gpu_pool[li][b, qi], s, wl.block_size, wl.cand_blocks, tag)
                elif plan.mode == "reindex":
                    pool = None if plan.source < 0 else gpu_pool[plan.source][b, qi]
                    ids = np.arange(n_vis) if pool is None else oc.pool_domain(pool, wl.block_size, n_vis)
                    s = oc.indexer_scores(spec.q_idx[i, qi], spec.head_w[i, qi], cache.idx_rows(ids)) if len(ids) else np.zeros(0)
                    summary["tie_diffs"] += check_index_set(top, ids, s, wl.topk, tag)
                else:
                    assert np.array_equal(top, gpu_topk[plan.source][b, qi]), f"{tag}: Reuse indices differ from source"
                rows = oc.gather_rows(cache, top, spec.swa[i], int(spec.swa_first[i]), t, wl.window)
                o, p, ls = oc.attention(spec.q[i, qi], t, rows, wl.d_rope, driver.rope_cfg(wl))
                err, rl2 = check_outputs(out[b, qi], o, wl, tag)
                summary["max_abs"] = max(summary["max_abs"], err)
                summary["rel_l2"] = max(summary["rel_l2"], rl2)
                assert np.allclose(lse[b, qi], ls, atol=2e-2 if wl.act == "bf16" else 1e-5), f"{tag}: lse"
    return summary


def compare_cache_rows(step, cache, b, ids):
    """GPU-written rows `ids` of sequence b vs the oracle's stored bytes (main KV and indexer K): exact."""
    wl = step.wl
    ids = np.asarray(ids, dtype=np.int64)
    main_ref = cache.main_raw_rows(ids) if hasattr(cache, "main_raw_rows") else {k: v[ids] for k, v in cache.main_raw.items()}
    idx_ref = {k: v[ids] for k, v in cache.idx_raw.items()}
    t_ids = torch.from_numpy(ids).to(step.cache.main.device)
    if wl.kv == "fp4":
        pairs = [(step.cache.main[b][t_ids], main_ref["codes"]), (step.cache.main_scale[b][t_ids], main_ref["scales"]),
                 (step.cache.idx[b][t_ids], idx_ref["codes"]), (step.cache.idx_scale[b][t_ids], idx_ref["scales"])]
        for got, ref in pairs:
            bad = np.count_nonzero(got.cpu().numpy() != ref)
            assert bad == 0, f"seq {b}: {bad} FP4 bytes differ on sampled rows"
    else:
        key = "bf16" if wl.kv == "bf16" else "f32"
        for got, ref in ((step.cache.main[b][t_ids], main_ref[key]), (step.cache.idx[b][t_ids], idx_ref[key])):
            g = got.cpu()
            g = g.view(torch.int16).numpy().view(np.uint16) if key == "bf16" else g.numpy()
            bad = np.count_nonzero(g != ref)
            assert bad == 0, f"seq {b}: {bad} {key} elements differ on sampled rows"
