"""The cross-layer plan of a CSA2 model: which layers share a cache, and each
layer's mode — the oracle's statement of it.

TEST INFRASTRUCTURE ONLY (see the oracle package header).

Sources: zartbot's walkthrough (hn.213312.xyz), section 1.2 (compress ratios
[0, 0, 2 x 18, 1 x 20]; kv-source layers [2, 8, 14, 20]; index-source layers
[2, 8, 14, 20, 24, 28, 32, 36]; candidate-source layer 20), section 2.3.3
(an encoder block is one Full layer and five Reuse layers; the decoder's first
block opens with a Full layer that builds the HSI candidate pool, the next
blocks open with a Reindex layer that searches that pool), sections 3.3.1
and 3.3.3 (reuse flows only from earlier to later layers; a Reuse layer
follows the most recent layer that published an index).

Readings: a layer of ratio 0 keeps no compressed KV (window attention only);
the layers from one kv-source layer up to the next form its group (one
shared main KV and indexer K); inside a group each index-source layer opens a
block (the kv source itself is Full, the others Reindex) and the block's
remaining layers Reuse the block's opening layer.
"""
from __future__ import annotations

from dataclasses import dataclass

# the pages' schedule ([ZB] 1.2)
PAGES_RATIOS = (0, 0) + (2,) * 18 + (1,) * 20
PAGES_KV_SOURCES = (2, 8, 14, 20)
PAGES_INDEX_SOURCES = (2, 8, 14, 20, 24, 28, 32, 36)
PAGES_CANDIDATE_SOURCE = 20


@dataclass(frozen=True)
class PlannedLayer:
    group: int  # kv-source layer whose caches the layer uses (-1: window only)
    mode: str  # "window" | "full" | "reindex" | "reuse"
    source: int  # reindex: pool layer or -1; reuse: layer whose top-k is read; else -1
    make_pool: bool = False


def layer_plan(ratios, kv_sources, index_sources, candidate_source) -> list[PlannedLayer]:
    """Group and mode of every layer, built block by block as the pages describe the model."""
    kv_sources, index_sources = sorted(kv_sources), sorted(index_sources)
    plan: list[PlannedLayer | None] = [None] * len(ratios)
    for l, r in enumerate(ratios):
        if r == 0:
            plan[l] = PlannedLayer(-1, "window", -1)
    # groups: [kv source, next kv source) restricted to layers with compressed KV
    bounds = list(kv_sources) + [len(ratios)]
    for g, start in enumerate(kv_sources):
        stop = bounds[g + 1]
        members = [l for l in range(start, stop) if ratios[l] != 0]
        if any(ratios[l] != ratios[start] for l in members):
            raise ValueError(f"group of layer {start} mixes compress ratios")
        # blocks: each index-source layer of the group opens one
        openers = [l for l in members if l in index_sources]
        if start not in openers:
            raise ValueError(f"kv-source layer {start} is not an index source")
        for b, head in enumerate(openers):
            block_end = openers[b + 1] if b + 1 < len(openers) else stop
            for l in range(head, block_end):
                if ratios[l] == 0:
                    continue
                if l == start:
                    plan[l] = PlannedLayer(start, "full", -1, make_pool=(l == candidate_source))
                elif l == head:
                    plan[l] = PlannedLayer(start, "reindex", start if start == candidate_source else -1)
                else:
                    plan[l] = PlannedLayer(start, "reuse", head)
    if any(p is None for p in plan):
        missing = [l for l, p in enumerate(plan) if p is None]
        raise ValueError(f"layers {missing} have compressed KV but no earlier kv-source layer")
    return plan


def cache_bytes_per_token(plan, ratios, main_entry_bytes: float, index_entry_bytes: float) -> float:
    """Compressed-KV bytes stored per token: every group's main-KV and
    indexer-K entry, divided by its compress ratio ([ZB] 3.1 counts the
    global KV of the kv-source layers only)."""
    groups = sorted({p.group for p in plan if p.group >= 0})
    return sum((main_entry_bytes + index_entry_bytes) / ratios[g] for g in groups)
