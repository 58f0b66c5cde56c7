"""A CSA2 model's layers grouped by shared cache, from csa2_layer_plan.

Host-side marshalling only: the plan itself is derived by the library
(csa2_layer_plan) and each group runs as one csa2_layer_group call over its
own caches.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import binding as B


@dataclass(frozen=True)
class GroupLayer:
    layer: int      # layer number in the model
    mode: int       # B.FULL / B.REINDEX / B.REUSE
    source: int     # position of the source layer inside the group, or -1
    make_pool: bool


class ModelPlan:
    """Per-layer plan of a model and its cache groups (see csa2_layer_plan in csa2.h)."""

    def __init__(self, ratios, kv_sources, index_sources, candidate_source=-1):
        self.ratios = list(ratios)
        self.layers = B.csa2_layer_plan(self.ratios, list(kv_sources), list(index_sources), candidate_source)

    def window_only(self) -> list[int]:
        """Layers that keep no compressed KV (sliding-window attention only)."""
        return [l for l, (g, _, _, _) in enumerate(self.layers) if g < 0]

    def groups(self) -> dict[int, list[GroupLayer]]:
        """kv-source layer -> its group's layers in order, sources as positions in the group
        (the form csa2_layer_group takes)."""
        out: dict[int, list[GroupLayer]] = {}
        pos: dict[int, int] = {}
        for l, (g, mode, source, make_pool) in enumerate(self.layers):
            if g < 0:
                continue
            members = out.setdefault(g, [])
            pos[l] = len(members)
            members.append(GroupLayer(l, mode, pos[source] if source >= 0 else -1, bool(make_pool)))
        return out

    def ratio_of(self, group: int) -> int:
        return self.ratios[group]
