"""Run one CSA2 step of a workload through the oracle.

TEST INFRASTRUCTURE ONLY (see the oracle package header).

``inp`` is any object with the seeded-input interface (``wl`` plus
``latent(b, start, stop)``, ``pair_logits()``, ``w_ik()``, ``q(l)``,
``q_idx(l)``, ``head_w(l)``, ``swa(l)``); the driver reads arrays from it and
imports nothing from the product.

A step is: compress the new latent rows into the cache (the cache already
holds every earlier entry), then run the layer group for the queries at the
last ``n_q`` positions.
"""
from __future__ import annotations

import numpy as np

from . import csa2, formats


def rope_cfg(wl) -> csa2.Rope:
    """RoPE settings of a workload (base theta, YaRN factor and original length)."""
    return csa2.Rope(float(wl.rope_theta), float(wl.rope_factor), int(wl.rope_orig_len))


def dims_of(wl) -> csa2.Dims:
    return csa2.Dims(
        d=wl.d, d_rope=wl.d_rope, n_heads=wl.n_heads, n_idx_heads=wl.n_idx_heads, d_idx=wl.d_idx,
        topk=wl.topk, window=wl.window, block_size=wl.block_size, cand_blocks=wl.cand_blocks,
        ratio=wl.ratio, rope_theta=rope_cfg(wl),
    )


def build_cache(inp, b: int, stop_pos: int, chunk: int = 1 << 14) -> csa2.SeqCache:
    """Cache of sequence b holding every entry made from positions 0 .. stop_pos-1."""
    wl = inp.wl
    logits, w_ik = inp.pair_logits(), inp.w_ik()
    cache = csa2.SeqCache(wl.kv, wl.main_group, wl.idx_group, {}, {})
    chunk -= chunk % wl.ratio
    for p0 in range(0, stop_pos, chunk):
        p1 = min(stop_pos, p0 + chunk)
        _, main_raw, _, idx_raw, _ = csa2.make_entries(
            inp.latent(b, p0, p1), p0, logits, w_ik, wl.ratio, wl.d_rope, rope_cfg(wl), wl.kv,
            wl.main_group, wl.idx_group,
        )
        cache.append(main_raw, idx_raw)
    return cache


def layer_specs(inp, seqs) -> list:
    """Per-layer oracle specs holding the query-side tensors of sequences ``seqs``."""
    wl = inp.wl
    specs = []
    for li, plan in enumerate(wl.layers):
        swa, swa_first = inp.swa(li)
        if wl.swa == "fp8":  # E4M3 (FN) bytes: the window KV kept in FP8 ([ZB] 2.4.4)
            swa = formats.e4m3_decode(swa)
        specs.append(
            csa2.LayerSpec(
                mode=plan.mode, source=plan.source, make_pool=plan.make_pool,
                q=inp.q(li)[seqs].astype(np.float64), q_idx=inp.q_idx(li)[seqs].astype(np.float64),
                head_w=inp.head_w(li)[seqs].astype(np.float64), swa=swa[seqs].astype(np.float64),
                swa_first=swa_first[seqs],
            )
        )
    return specs


def run_step(inp, seqs=None, caches=None):
    """Oracle result of one step for sequences ``seqs`` (default: all).

    ``caches`` may pass prebuilt prior caches (entries from positions
    0 .. prior-1); the step's new entries are appended to copies of them.
    Returns (per-layer results of csa2.run_group, caches after the step).
    """
    wl = inp.wl
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    dims = dims_of(wl)
    out_caches = []
    for i, b in enumerate(seqs):
        if caches is None:
            cache = build_cache(inp, b, wl.prior)
        else:
            src = caches[i]
            cache = csa2.SeqCache(src.kv_fmt, src.main_group, src.idx_group,
                                  {k: v.copy() for k, v in src.main_raw.items()},
                                  {k: v.copy() for k, v in src.idx_raw.items()})
        if wl.new:
            _, main_raw, _, idx_raw, _ = csa2.make_entries(
                inp.latent(b, wl.prior, wl.context), wl.prior, inp.pair_logits(), inp.w_ik(), wl.ratio,
                wl.d_rope, rope_cfg(wl), wl.kv, wl.main_group, wl.idx_group,
            )
            cache.append(main_raw, idx_raw)
        out_caches.append(cache)
    q_pos = wl.q_positions()[seqs]
    n_entries = [c.n_entries for c in out_caches]
    results = csa2.run_group(dims, out_caches, n_entries, q_pos, layer_specs(inp, seqs))
    return results, out_caches


class LazyMainCache(csa2.SeqCache):
    """A sequence cache whose indexer K is stored in full but whose main-KV
    rows are made (compressed, rotated, stored) only when a row is read.

    Same arithmetic as build_cache; it only defers the main-KV rows, which a
    step reads for the few kept entries, so very long contexts fit in memory.
    """

    def __init__(self, inp, b: int, stop_pos: int, chunk: int = 1 << 14):
        wl = inp.wl
        super().__init__(wl.kv, wl.main_group, wl.idx_group, {}, {})
        self.inp, self.b = inp, b
        self._n = stop_pos // wl.ratio
        logits, w_ik = inp.pair_logits(), inp.w_ik()
        chunk -= chunk % wl.ratio
        for p0 in range(0, stop_pos, chunk):
            p1 = min(stop_pos, p0 + chunk)
            e = csa2.compress(inp.latent(b, p0, p1), logits, wl.ratio)
            j = p0 // wl.ratio + np.arange(e.shape[0])
            e_hat = csa2.rope(e, csa2.entry_position(j, wl.ratio), wl.d_rope, rope_cfg(wl))
            _, idx_raw = formats_store(e_hat @ np.asarray(w_ik, dtype=np.float64), wl.kv, wl.idx_group)
            for key, arr in idx_raw.items():
                self.idx_raw.setdefault(key, []).append(arr)
        self.idx_raw = {k: np.concatenate(v) for k, v in self.idx_raw.items()}

    @property
    def n_entries(self) -> int:
        return self._n

    def main_raw_rows(self, ids, fetch: int = 4096) -> dict:
        """Raw stored main-KV parts of the given entries (latent read in aligned runs of `fetch` positions)."""
        wl = self.inp.wl
        ids = np.asarray(ids, dtype=np.int64)
        fetch -= fetch % wl.ratio
        rows = {}
        for blk in np.unique(ids * wl.ratio // fetch):
            p0 = int(blk) * fetch
            sel = ids[(ids * wl.ratio // fetch) == blk]
            lat = self.inp.latent(self.b, p0, p0 + fetch)
            for j in np.unique(sel):
                q0 = int(j) * wl.ratio - p0
                e = csa2.compress(lat[q0 : q0 + wl.ratio], self.inp.pair_logits(), wl.ratio)
                e_hat = csa2.rope(e, csa2.entry_position(np.array([j]), wl.ratio), wl.d_rope, rope_cfg(wl))
                rows[int(j)] = formats_store(e_hat, wl.kv, wl.main_group)[1]
        keys = rows[int(ids[0])].keys() if len(ids) else []
        return {k: np.concatenate([rows[int(j)][k] for j in ids]) for k in keys}

    def main_rows(self, ids) -> np.ndarray:
        ids = np.asarray(ids, dtype=np.int64)
        if len(ids) == 0:
            return np.zeros((0, self.inp.wl.d))
        raw = self.main_raw_rows(ids)
        return self._decode(raw, np.arange(len(ids)), self.main_group)


def formats_store(x, fmt, group):
    from . import formats

    return formats.store(x, fmt, group)
