"""Global-KV bytes per token from the FP4 codec's own byte counts — the oracle.

TEST INFRASTRUCTURE ONLY (see the oracle package header).

[ZB] 3.1 (zartbot walkthrough, hn.213312.xyz, "why the KV is 890 B"): the
HBM-resident global KV of a token is the main-KV entry plus the indexer-K
entry of every KV-source layer, divided by that layer's compress ratio.  The
sources are encoder layers 2, 8, 14 at ratio 2 and decoder layer 20 at ratio
1 ([ZB] 1.2 kv_source_layers).  Entry sizes come from formats.fp4_entry_bytes,
i.e. from what the codec actually emits.
"""
from __future__ import annotations

from fractions import Fraction

from . import formats

# (layer, compress ratio) of every layer that owns a main KV and an indexer K.
KV_SOURCES = ((2, 2), (8, 2), (14, 2), (20, 1))


def bytes_per_token(main_channels=512, idx_channels=128, main_group=16, idx_group=32, sources=KV_SOURCES) -> Fraction:
    """Stored bytes per token summed over the KV-source layers (exact fraction)."""
    main = formats.fp4_entry_bytes(main_channels, main_group)
    idx = formats.fp4_entry_bytes(idx_channels, idx_group)
    return sum((Fraction(main + idx, ratio) for _, ratio in sources), Fraction(0))


def chain_from_entry(main_entry_bytes: int, idx_entry_bytes: int, sources) -> Fraction:
    """Bytes per token for given per-entry sizes and (layer, ratio) sources."""
    return sum((Fraction(main_entry_bytes + idx_entry_bytes, r) for _, r in sources), Fraction(0))
