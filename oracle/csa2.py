"""CSA2 hot path, stated plainly in float64 — the oracle.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
does, and nothing here is shared with the HIP path.

Sources (all web pages about the DeepSeek-V4.1-Flash technical report):

* [ZB]   zartbot's walkthrough of the report as rendered on hn.213312.xyz,
         sections 1.1-3.3.3 (Chinese).
* [ELPH] elph.ru, "DeepSeek-V4.1 Flash: Squeezing the KV Cache Fourfold for
         Long Context", section "Three dimensions of compression".
* [36KR] eu.36kr.com, "What 'black technologies' does DeepSeek V4.1 Flash
         adopt?", headings "CSA2: Three compression dimensions ..." and "FP4
         and Bounded Replay".

The pages print no formulas for the compressor, the indexer score or the
attention; each step below states the reading it takes.  Every floating-point
step runs in float64; rounding happens only where a value is stored in the
cache (main KV, indexer K).

Notation: d latent width (= query head width), d_rope trailing rotary
channels, r compress ratio, H query heads, Hi indexer heads of width di,
k top-k, W window, beta HSI block size, kappa HSI candidate blocks.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import formats

# --------------------------------------------------------------------------
# a1. Compressor
# --------------------------------------------------------------------------


def pair_weights(logits: np.ndarray) -> np.ndarray:
    """Per-channel merge weights: softmax over the r positions of each channel.

    [ZB] 1.1 and [ELPH]: the encoder merges two adjacent positions into one
    entry with channel-wise learned weights.  Reading: static learned logits
    A[r, d], normalised by a softmax over the r merged positions, channel by
    channel.  logits: [r, d] -> weights [r, d].
    """
    a = np.asarray(logits, dtype=np.float64)
    e = np.exp(a - a.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def compress(latent: np.ndarray, logits: np.ndarray | None, ratio: int) -> np.ndarray:
    """Merge each run of ``ratio`` adjacent latent rows into one entry.

    [ZB] 2.3.1: ratio 2 in the causal encoder, ratio 1 in the decoder, no
    overlapping windows.  latent [T, d] with T a multiple of ratio ->
    entries [T/ratio, d]: e_j[c] = sum_i a[i, c] * X[ratio*j + i, c].
    Ratio 1 returns the latent unchanged.

    The weights sum to 1, so the sum is evaluated as the last row plus the
    weighted differences of the others from it: the same value, and exact
    when the merged rows agree (a stored code then is that of the row itself,
    also when the row sits on a rounding tie of the storage format).
    """
    x = np.asarray(latent, dtype=np.float64)
    t, d = x.shape
    if t % ratio:
        raise ValueError("compress: row count must be a multiple of the ratio")
    if ratio == 1:
        return x.copy()
    a = pair_weights(logits)
    groups = x.reshape(t // ratio, ratio, d)
    last = groups[:, ratio - 1, :]
    out = np.zeros((t // ratio, d))
    for i in range(ratio - 1):
        out += a[i][None, :] * (groups[:, i, :] - last)
    return out + last


def entry_position(j: np.ndarray | int, ratio: int):
    """Token position an entry is rotated at: the last position it covers.

    Reading (the pages are silent): entry j covers positions ratio*j ..
    ratio*j + ratio - 1 and carries the position of the last one.
    """
    return ratio * np.asarray(j) + ratio - 1


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Rope:
    """RoPE settings: base theta, and the YaRN extension ([ZB] 1.2: original
    length 65536, factor 16).  factor <= 1 is plain RoPE."""

    theta: float = 10000.0
    factor: float = 1.0
    orig_len: int = 0


def _rope_cfg(theta) -> Rope:
    return theta if isinstance(theta, Rope) else Rope(float(theta))


def rope_freqs(theta, d_rope: int) -> np.ndarray:
    """Angle per position of rotary pair m = 0 .. d_rope/2 - 1.

    Plain: f_m = theta^(-2m/d_rope).  YaRN (the pages name only its original
    length and factor; the interpolation is the YaRN paper's "NTK-by-parts",
    Peng et al. 2023, with its alpha = 1, beta = 32): with r_m the number of
    wavelengths 2 pi / f_m that fit the original length L, a pair keeps f_m
    when r_m >= 32, turns at f_m / s when r_m <= 1, and blends linearly in r
    between the two.  **Parity unpinned by the pages** beyond factor and L.
    """
    cfg = _rope_cfg(theta)
    m = np.arange(d_rope // 2, dtype=np.float64)
    freq = np.power(float(cfg.theta), -2.0 * m / d_rope)
    if cfg.factor > 1.0:
        r = cfg.orig_len / (2.0 * np.pi / freq)
        g = np.clip((r - 1.0) / (32.0 - 1.0), 0.0, 1.0)
        freq = (1.0 - g) * (freq / cfg.factor) + g * freq
    return freq


def logit_temperature(theta) -> float:
    """YaRN's attention temperature: logits times (0.1 ln s + 1)^2 (1 without YaRN)."""
    cfg = _rope_cfg(theta)
    return (0.1 * np.log(cfg.factor) + 1.0) ** 2 if cfg.factor > 1.0 else 1.0


def rope(x: np.ndarray, pos, d_rope: int, theta) -> np.ndarray:
    """Rotate the trailing ``d_rope`` channels of ``x[..., d]`` by position ``pos``.

    [ZB] 1.2 lists 64 rotary dims inside the 512-d latent, theta 10000; the
    cache is stored after rotation ([ZB] 2.4.4).  Reading: the rotary channels
    are the last d_rope; pair m holds channels (c0 + 2m, c0 + 2m + 1) with
    c0 = d - d_rope and turns by angle pos * f_m (rope_freqs; ``theta`` is a
    base or a Rope).  ``pos`` broadcasts against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    c0 = d - d_rope
    freq = rope_freqs(theta, d_rope)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * freq
    cos, sin = np.cos(phi), np.sin(phi)
    out = x.copy()
    xe = x[..., c0::2]
    xo = x[..., c0 + 1 :: 2]
    out[..., c0::2] = xe * cos - xo * sin
    out[..., c0 + 1 :: 2] = xe * sin + xo * cos
    return out


# --------------------------------------------------------------------------
# a1/a2/a7. Cache writes
# --------------------------------------------------------------------------


@dataclass
class SeqCache:
    """One sequence's shared caches (main KV and indexer K) as stored.

    ``main_raw`` / ``idx_raw`` hold the raw stored parts of every entry (see
    formats.store); rows are decoded to float64 on demand.
    """

    kv_fmt: str
    main_group: int
    idx_group: int
    main_raw: dict
    idx_raw: dict

    @property
    def n_entries(self) -> int:
        return len(next(iter(self.main_raw.values())))

    def _decode(self, raw: dict, ids, group: int) -> np.ndarray:
        if self.kv_fmt == "f32":
            return raw["f32"][ids].astype(np.float64)
        if self.kv_fmt == "bf16":
            return formats.bf16_decode(raw["bf16"][ids])
        return formats.fp4_decode(raw["codes"][ids], raw["scales"][ids], group)

    def main_rows(self, ids) -> np.ndarray:
        return self._decode(self.main_raw, ids, self.main_group)

    def idx_rows(self, ids) -> np.ndarray:
        return self._decode(self.idx_raw, ids, self.idx_group)

    def append(self, main_raw: dict, idx_raw: dict) -> None:
        for dst, src in ((self.main_raw, main_raw), (self.idx_raw, idx_raw)):
            for key, arr in src.items():
                dst[key] = np.concatenate([dst[key], arr]) if key in dst else arr


def make_entries(
    latent: np.ndarray,
    first_pos: int,
    logits: np.ndarray | None,
    w_ik: np.ndarray,
    ratio: int,
    d_rope: int,
    theta: float,
    kv_fmt: str,
    main_group: int = 32,
    idx_group: int = 32,
) -> tuple[np.ndarray, dict, np.ndarray, dict, np.ndarray]:
    """Compress, rotate and store the entries made from ``latent``.

    latent [T, d] holds positions first_pos .. first_pos + T - 1 (first_pos a
    multiple of ratio).  Steps, in the pages' order:

    1. merge adjacent rows ([ZB] 2.3.1);
    2. rotate entry j at its position ([ZB] 2.4.4: quantised after RoPE);
    3. store the main KV row ([ZB] 2.4.4: FP4 main KV);
    4. indexer K = rotated entry times W_ik, 512 -> 128 ([ZB] 2.3.1: the
       indexer K is projected from the main KV).  Reading: the projection
       takes the unrounded rotated entry;
    5. store the indexer K row.

    Returns (main values, main raw, idx values, idx raw, rotated entries).
    """
    if first_pos % ratio:
        raise ValueError("make_entries: first position must be a multiple of the ratio")
    e = compress(latent, logits, ratio)
    j = first_pos // ratio + np.arange(e.shape[0])
    e_hat = rope(e, entry_position(j, ratio), d_rope, theta)
    main, main_raw = formats.store(e_hat, kv_fmt, main_group)
    kappa = e_hat @ np.asarray(w_ik, dtype=np.float64)
    idx, idx_raw = formats.store(kappa, kv_fmt, idx_group)
    return main, main_raw, idx, idx_raw, e_hat


# --------------------------------------------------------------------------
# Visibility
# --------------------------------------------------------------------------


def visible_entries(n_entries: int, t: int, ratio: int) -> int:
    """Number of entries query position t may read: j visible iff ratio*j + ratio - 1 <= t.

    Reading (the pages only say the attention is causal): an entry becomes
    visible once every position it covers is at or before t.  Entries are a
    prefix 0 .. n-1.
    """
    if t + 1 <= 0:
        return 0
    return int(min(n_entries, (t + 1) // ratio))


def window_positions(t: int, window: int) -> np.ndarray:
    """Positions of the sliding window of query t: max(0, t-W+1) .. t ([ZB] 1.2: window 128)."""
    return np.arange(max(0, t - window + 1), t + 1)


# --------------------------------------------------------------------------
# a3. Indexer score
# --------------------------------------------------------------------------


def indexer_scores(q_idx: np.ndarray, head_w: np.ndarray, idx_rows: np.ndarray) -> np.ndarray:
    """Indexer score of each row: s_j = sum_h w_h * max(0, q_idx[h] . K_j).

    [ZB] 2.3.1: the lightweight indexer scores main-KV entries with indexer Q
    and K; [ZB] 1.2: 32 heads of width 128.  The pages give no formula;
    reading: a per-head ReLU of the dot product, weighted by the query's own
    head weights and summed over heads.
    q_idx [Hi, di], head_w [Hi], idx_rows [n, di] -> [n].
    """
    dots = np.asarray(idx_rows, dtype=np.float64) @ np.asarray(q_idx, dtype=np.float64).T
    return np.maximum(dots, 0.0) @ np.asarray(head_w, dtype=np.float64)


# --------------------------------------------------------------------------
# a4. Top-k and HSI
# --------------------------------------------------------------------------


def rank_order(scores: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Positions of (score, id) pairs ordered by descending score, then ascending id.

    Reading (ties are not discussed on the pages): equal scores go to the
    lower index.
    """
    return np.lexsort((np.asarray(ids), -np.asarray(scores, dtype=np.float64)))


def topk_select(scores: np.ndarray, ids: np.ndarray, k: int) -> np.ndarray:
    """The k best ids of a domain, emitted ascending and padded with -1 to length k.

    [ZB] 1.2: index_topk 512.  With fewer than k candidates every candidate
    is kept.
    """
    order = rank_order(scores, ids)[:k]
    chosen = np.sort(np.asarray(ids)[order])
    out = np.full(k, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out


def block_maxima(scores: np.ndarray, beta: int) -> np.ndarray:
    """Max score of each block [beta*b, beta*b + beta) over the given (visible) prefix."""
    n = len(scores)
    nb = -(-n // beta)
    return np.array([np.max(scores[b * beta : min(n, b * beta + beta)]) for b in range(nb)])


def hsi_pool(scores: np.ndarray, beta: int, kappa: int) -> np.ndarray:
    """HSI candidate pool: kappa block ids, ascending, padded with -1.

    [ZB] 2.3.4: the Full layer reduces its full scores to a per-block maximum
    over blocks of 8, keeps the highest 2048 blocks, always including the
    block that holds the newest visible position, and expands them into a
    fixed-size pool.  Readings: blocks are aligned [8b, 8b+8); a partial last
    block uses only its visible entries; the forced block counts toward the
    kappa blocks; block ties go to the lower block id.
    ``scores`` covers visible entries 0 .. n_vis-1.
    """
    n_vis = len(scores)
    out = np.full(kappa, -1, dtype=np.int64)
    if n_vis == 0:
        return out
    bmax = block_maxima(scores, beta)
    nb = len(bmax)
    if nb <= kappa:
        out[:nb] = np.arange(nb)
        return out
    forced = (n_vis - 1) // beta
    others = np.array([b for b in range(nb) if b != forced])
    order = rank_order(bmax[others], others)[: kappa - 1]
    chosen = np.sort(np.concatenate([[forced], others[order]]))
    out[:] = chosen
    return out


def pool_domain(pool: np.ndarray, beta: int, n_vis: int) -> np.ndarray:
    """Entry ids a pool covers that are visible, ascending (a Reindex layer's search domain)."""
    ids = [j for b in pool if b >= 0 for j in range(b * beta, b * beta + beta) if j < n_vis]
    return np.array(sorted(ids), dtype=np.int64)


# --------------------------------------------------------------------------
# a5. Sparse attention with the sliding window
# --------------------------------------------------------------------------


def attention(q: np.ndarray, t: int, rows: np.ndarray, d_rope: int, theta):
    """Softmax attention of all heads of one query over the concatenated rows.

    [ZB] 2.2.2: global KV (sparse) and local KV (window) are concatenated and
    scored together with Q; [ZB] 3.3.1: key equals value, so the output is a
    convex combination of the rows.  Readings: the query is rotated at its
    own position t, logits are scaled by 1/sqrt(d), one softmax runs over all
    rows (no de-duplication, no sink), and V is the full stored row.  With
    YaRN (``theta`` a Rope with factor > 1) the logits also take its
    temperature (logit_temperature).
    q [H, d], rows [n, d] -> (O [H, d], P [H, n], lse [H]) with lse the natural
    log of the softmax denominator of the scaled logits.
    """
    d = q.shape[-1]
    q_hat = rope(q, t, d_rope, theta)
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        raise ValueError("attention: no rows to attend to")
    logits = (q_hat @ rows.T) * (logit_temperature(theta) / np.sqrt(d))
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=1, keepdims=True)
    p = e / den
    out = p @ rows
    lse = (m + np.log(den))[:, 0]
    return out, p, lse


def grouped_out_proj(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """The grouped low-rank output projection after the attention (zartbot
    walkthrough, section 1.2: o_lora_rank 1024 in o_groups 8).

    ``x`` [n, G*K]: attention output rows, the heads' outputs concatenated;
    ``w`` [G, R, K]: group g's R outputs, each a weight row over the group's
    own K channels.  Group g maps channels [g K, g K + K) of a row to outputs
    [g R, g R + R): y[:, gR:gR+R] = x[:, gK:gK+K] w[g]^T.  float64.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    G, R, K = w.shape
    if x.shape[1] != G * K:
        raise ValueError(f"x has {x.shape[1]} channels, groups need {G} x {K}")
    y = np.empty((x.shape[0], G * R))
    for g in range(G):
        y[:, g * R:(g + 1) * R] = x[:, g * K:(g + 1) * K] @ w[g].T
    return y


def gather_rows(cache: "SeqCache", topk: np.ndarray, swa: np.ndarray, swa_first: int, t: int, window: int):
    """Rows one query reads: selected main-KV rows (skipping -1), then its window rows.

    Window rows outside the supplied SWA buffer are skipped.
    """
    ids = np.array([j for j in topk if j >= 0], dtype=np.int64)
    sel = cache.main_rows(ids) if len(ids) else np.zeros((0, swa.shape[-1]))
    win_pos = [p for p in window_positions(t, window) if 0 <= p - swa_first < len(swa)]
    win = np.asarray(swa, dtype=np.float64)[np.array(win_pos, dtype=np.int64) - swa_first] if win_pos else np.zeros((0, swa.shape[-1]))
    return np.concatenate([sel, win])


# --------------------------------------------------------------------------
# a6. One query through a layer, and a group of layers
# --------------------------------------------------------------------------


@dataclass
class Dims:
    d: int
    d_rope: int
    n_heads: int
    n_idx_heads: int
    d_idx: int
    topk: int
    window: int
    block_size: int = 8
    cand_blocks: int = 2048
    ratio: int = 1
    rope_theta: "float | Rope" = 10000.0  # a base, or a Rope with YaRN settings


def full_scores(cache: "SeqCache", n_vis: int, q_idx, head_w, chunk: int = 1 << 16) -> np.ndarray:
    """Indexer scores of visible entries 0 .. n_vis-1, decoding the stored rows chunk by chunk."""
    parts = [indexer_scores(q_idx, head_w, cache.idx_rows(slice(c, min(n_vis, c + chunk))))
             for c in range(0, n_vis, chunk)]
    return np.concatenate(parts) if parts else np.zeros(0)


def full_query(dims: Dims, cache: "SeqCache", n_entries: int, t: int, q_idx, head_w, make_pool: bool):
    """Full mode for one query: score every visible entry, take the top-k, optionally the HSI pool.

    [ZB] 2.3.2 / [36KR]: Full runs the complete indexer over all visible
    entries.  [ZB] 2.3.4: the Full layer's own top-k comes from its full
    scores; the pool is built from the same scores.
    Returns (topk ids, pool or None, scores over visible entries).
    """
    n_vis = visible_entries(n_entries, t, dims.ratio)
    ids = np.arange(n_vis)
    s = full_scores(cache, n_vis, q_idx, head_w)
    top = topk_select(s, ids, dims.topk)
    pool = hsi_pool(s, dims.block_size, dims.cand_blocks) if make_pool else None
    return top, pool, s


def reindex_query(dims: Dims, cache: "SeqCache", n_entries: int, t: int, q_idx, head_w, pool):
    """Reindex mode for one query: rescore the shared indexer K with this layer's own indexer Q.

    [ZB] 2.3.2: reuse main KV and indexer K, recompute the top-k with the
    layer's own indexer Q.  [ZB] 2.3.4: in the decoder the search domain is
    the Full layer's HSI pool.  ``pool`` None searches all visible entries.
    """
    n_vis = visible_entries(n_entries, t, dims.ratio)
    ids = np.arange(n_vis) if pool is None else pool_domain(pool, dims.block_size, n_vis)
    s = indexer_scores(q_idx, head_w, cache.idx_rows(ids)) if len(ids) else np.zeros(0)
    return topk_select(s, ids, dims.topk), s, ids


@dataclass
class LayerSpec:
    """One layer of a group. mode: "full" | "reindex" | "reuse".

    source: reindex -> index of the earlier Full layer whose pool is searched
    (or -1 for all visible entries); reuse -> index of the earlier layer whose
    top-k is read.  Per-query tensors are indexed [b][qi].
    """

    mode: str
    source: int = -1
    make_pool: bool = False
    q: np.ndarray | None = None  # [B, nq, H, d]
    q_idx: np.ndarray | None = None  # [B, nq, Hi, di]
    head_w: np.ndarray | None = None  # [B, nq, Hi]
    swa: np.ndarray | None = None  # [B, n_swa, d]
    swa_first: np.ndarray | None = None  # [B]


def run_group(dims: Dims, caches: list, n_entries: list, q_pos: np.ndarray, layers: list):
    """Run a group of layers that share one main KV and indexer K.

    [ZB] 3.2 access table: Full writes main KV, indexer K and top-k; Reindex
    reads main KV and indexer K and rewrites the top-k; Reuse reads main KV
    and the top-k and never touches the indexer K.  Every layer keeps its own
    query and window ([36KR] "CSA2 ...").  [ZB] 3.3.1: reuse only flows from
    earlier to later layers.

    caches[b] is a SeqCache (already holding this step's new entries);
    q_pos [B, nq].  Returns per layer a dict with "topk" [B, nq, k],
    "pool" [B, nq, kappa] or None, "out" [B, nq, H, d], "lse" [B, nq, H],
    "probs" (list of P arrays).
    """
    B, nq = q_pos.shape
    results = []
    for li, L in enumerate(layers):
        if L.mode != "full" and not (0 <= L.source < li) and not (L.mode == "reindex" and L.source == -1):
            raise ValueError("run_group: a Reindex/Reuse source must be an earlier layer")
        topk = np.full((B, nq, dims.topk), -1, dtype=np.int64)
        pool = np.full((B, nq, dims.cand_blocks), -1, dtype=np.int64) if (L.mode == "full" and L.make_pool) else None
        out = np.zeros((B, nq, dims.n_heads, dims.d))
        lse = np.zeros((B, nq, dims.n_heads))
        probs = []
        for b in range(B):
            cache = caches[b]
            for qi in range(nq):
                t = int(q_pos[b, qi])
                if L.mode == "full":
                    top, pl, _ = full_query(
                        dims, cache, n_entries[b], t, L.q_idx[b, qi], L.head_w[b, qi], L.make_pool
                    )
                    if pool is not None:
                        pool[b, qi] = pl
                elif L.mode == "reindex":
                    src_pool = None if L.source == -1 else results[L.source]["pool"]
                    if L.source != -1 and src_pool is None:
                        raise ValueError("run_group: Reindex source has no pool")
                    top, _, _ = reindex_query(
                        dims, cache, n_entries[b], t, L.q_idx[b, qi], L.head_w[b, qi],
                        None if src_pool is None else src_pool[b, qi],
                    )
                elif L.mode == "reuse":
                    top = results[L.source]["topk"][b, qi].copy()
                else:
                    raise ValueError(f"unknown mode {L.mode!r}")
                topk[b, qi] = top
                rows = gather_rows(cache, top, L.swa[b], int(L.swa_first[b]), t, dims.window)
                o, p, ls = attention(L.q[b, qi], t, rows, dims.d_rope, dims.rope_theta)
                out[b, qi] = o
                lse[b, qi] = ls
                probs.append(p)
        results.append({"topk": topk, "pool": pool, "out": out, "lse": lse, "probs": probs})
    return results
