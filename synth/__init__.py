"""Seeded synthetic inputs for the CSA2 workloads.

This module only draws random numbers and rounds them to the activation
dtype; it holds none of the method's arithmetic.  Both the oracle-side tests
and the GPU side consume exactly the arrays it returns.

Every tensor gets its own PCG64 stream, keyed by (seed, workload, tensor,
layer, sequence, chunk), so a test can regenerate one sequence or one chunk
of a long latent without drawing the rest.

Distributions (the pages give none; the plainest choice for trained
activations at unit scale): latent, queries, indexer queries, head weights,
compressor logits and window rows are N(0, 1); the indexer-K projection W_ik
is N(0, 1/d) (standard deviation 1/sqrt(fan_in)); FP8 window rows are drawn
as E4M3 code bytes; the output projection's inputs are described at
oproj_inputs.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 4096  # latent rows per generated chunk


@dataclass(frozen=True)
class LayerPlan:
    mode: str  # "full" | "reindex" | "reuse"
    source: int = -1
    make_pool: bool = False


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    ratio: int
    d: int
    d_rope: int
    n_heads: int
    n_idx_heads: int
    d_idx: int
    topk: int
    window: int
    act: str  # activation dtype: "f32" | "bf16"
    kv: str  # cache dtype: "f32" | "bf16" | "fp4"
    prior: int  # latent positions already compressed into the cache
    new: int  # latent positions compressed by the step itself
    n_q: int  # queries per sequence, at the last n_q positions
    layers: tuple = (LayerPlan("full"),)
    block_size: int = 8
    cand_blocks: int = 2048
    main_group: int = 32
    idx_group: int = 32
    rope_theta: float = 10000.0
    rope_factor: float = 1.0  # YaRN factor (1 = plain RoPE)
    rope_orig_len: int = 0  # YaRN original context length
    swa: str = "act"  # window-row storage: "act" (the activation dtype) or "fp8" (E4M3 bytes)
    swa_replay: bool = False  # window buffer limited to the queries' own segment (bounded replay)
    description: str = ""

    @property
    def context(self) -> int:
        return self.prior + self.new

    @property
    def capacity(self) -> int:
        return self.context // self.ratio

    @property
    def n_prior_entries(self) -> int:
        return self.prior // self.ratio

    def q_positions(self) -> np.ndarray:
        t = np.arange(self.context - self.n_q, self.context, dtype=np.int32)
        return np.broadcast_to(t, (self.batch, self.n_q)).copy()

    def swa_span(self) -> tuple[int, int]:
        """First window position held in the window buffer and its number of rows
        per sequence: every row the queries' windows reach, or with bounded
        replay only the queries' own segment."""
        t0 = self.context - self.n_q
        first = t0 if self.swa_replay else max(0, t0 - self.window + 1)
        return first, self.context - first


_PROD = dict(d=512, d_rope=64, n_heads=64, n_idx_heads=32, d_idx=128, topk=512, window=128)

WORKLOADS = {
    # The five workloads the measurements are quoted on.
    "tiny_encoder": Workload(
        "tiny_encoder", batch=1, ratio=2, d=64, d_rope=16, n_heads=8, n_idx_heads=4, d_idx=32,
        topk=64, window=16, act="f32", kv="f32", prior=1008, new=16, n_q=16,
        description="tiny encoder layer, fp32: 1024 positions at ratio 2 (512 entries), "
        "causal decode of the last 16 queries",
    ),
    "decode_32k": Workload(
        "decode_32k", batch=16, ratio=1, **_PROD, act="bf16", kv="bf16", prior=32767, new=1, n_q=1,
        description="decoder-layer decode, bf16: 16 sequences x 32768 context, ratio 1, Full",
    ),
    "prefill_128k": Workload(
        "prefill_128k", batch=1, ratio=2, **_PROD, act="bf16", kv="bf16", prior=131072, new=4096, n_q=4096,
        description="encoder chunked prefill, bf16: 131072 prior positions at ratio 2, "
        "a chunk of 4096 causal queries",
    ),
    "group_256k": Workload(
        "group_256k", batch=4, ratio=1, **_PROD, act="bf16", kv="bf16", prior=262143, new=1, n_q=1,
        layers=(LayerPlan("full", make_pool=True), LayerPlan("reindex", 0), LayerPlan("reindex", 0),
                LayerPlan("reuse", 2)),
        description="cross-layer group decode, bf16: 4 x 262144, Full + Reindex + Reindex + Reuse(3rd)",
    ),
    "fp4_1m": Workload(
        "fp4_1m", batch=2, ratio=1, **_PROD, act="bf16", kv="fp4", prior=1048575, new=1, n_q=1,
        layers=(LayerPlan("full", make_pool=True),), main_group=32, idx_group=32,
        description="long-context decode with FP4 KV (E2M1, one E4M3 scale per 32): 2 x 1048576, HSI",
    ),
}

# Larger decode batches of the same shape (throughput as the batch grows;
# measured, not parity cases: the 32K case at batch 16 covers the kernels)
WORKLOADS["decode_32k_b64"] = replace(
    WORKLOADS["decode_32k"], name="decode_32k_b64", batch=64,
    description="decoder-layer decode, bf16: 64 sequences x 32768 context, ratio 1, Full")

# The encoder macro-block: one Full layer that writes the cache and the
# top-k, then five Reuse layers that attend with their own queries over the
# same kept entries (zartbot walkthrough, section 2.3.3), on the chunked
# prefill shape.
ENCODER_BLOCK = (LayerPlan("full"),) + (LayerPlan("reuse", 0),) * 5
WORKLOADS["encoder_block_128k"] = replace(
    WORKLOADS["prefill_128k"], name="encoder_block_128k", layers=ENCODER_BLOCK,
    description="encoder macro-block in chunked prefill, bf16: 131072 prior positions at ratio 2, a chunk of "
    "4096 causal queries, 1 Full + 5 Reuse layers",
)

# The pages' storage format for the 1M decode: FP4 main KV with one E4M3 scale
# per 16 channels (288 bytes per entry), FP4 indexer K with one per 32 (68
# bytes), and the window KV kept in FP8 (zartbot walkthrough, section 2.4.4).
WORKLOADS["fp4_1m_pages"] = replace(
    WORKLOADS["fp4_1m"], name="fp4_1m_pages", main_group=16, swa="fp8",
    description="long-context decode in the pages' storage format: 2 x 1048576, FP4 main KV per 16 channels, "
    "FP4 indexer K per 32, FP8 (E4M3) window rows, HSI",
)

# The 1M decode in the pages' storage format with their RoPE extension: YaRN
# from an original length of 65536 by a factor of 16, i.e. to 1048576
# positions (zartbot walkthrough, section 1.2).
WORKLOADS["fp4_1m_yarn"] = replace(
    WORKLOADS["fp4_1m_pages"], name="fp4_1m_yarn", rope_factor=16.0, rope_orig_len=65536,
    description="long-context decode, pages' storage format, YaRN RoPE (65536 x 16): 2 x 1048576, HSI",
)

# Decoder-side chunked prefill: ratio 1, every query of the chunk builds its
# own HSI pool in the Full layer and the Reindex layers rescore each query's
# pool with their own indexer queries (zartbot walkthrough, sections 2.3.3
# and 2.3.4: the decoder's first layer is Full and builds the candidate pool,
# the following ones Reindex inside it).
DECODER_PREFILL = (LayerPlan("full", make_pool=True), LayerPlan("reindex", 0), LayerPlan("reindex", 0))
WORKLOADS["decoder_prefill_64k"] = replace(
    WORKLOADS["decode_32k"], name="decoder_prefill_64k", batch=1, prior=65536, new=4096, n_q=4096,
    layers=DECODER_PREFILL,
    description="decoder chunked prefill, bf16: 65536 prior entries at ratio 1, a chunk of 4096 causal queries, "
    "Full with per-query HSI pools + 2 Reindex layers",
)

# The decoder's cache group in the pages' schedule (zartbot walkthrough 1.2 and
# 2.3.3; csa2_layer_plan derives it): layer 20 Full with the HSI pool, three
# Reuse layers, then four blocks of a Reindex layer over the pool and three
# Reuse layers of it (positions inside the group).
DECODER_GROUP = (LayerPlan("full", make_pool=True),) + (LayerPlan("reuse", 0),) * 3 + sum(
    ((LayerPlan("reindex", 0),) + (LayerPlan("reuse", 4 * i),) * 3 for i in range(1, 5)), ())

# Decoder SWA bounded replay (zartbot walkthrough 2.2.2; 36Kr "FP4 and
# Bounded Replay"): after an early-exit prefill only the last n_win = 128
# prompt positions run through the decoder, each attending to its kept
# entries and to window rows inside the replayed segment only.  The 64K
# prompt's decoder group, for the 128 replayed queries.
WORKLOADS["replay_64k"] = replace(
    WORKLOADS["decode_32k"], name="replay_64k", batch=1, prior=65536 - 128, new=128, n_q=128,
    layers=DECODER_GROUP, swa_replay=True,
    description="decoder SWA bounded replay, bf16: the last 128 positions of a 65536-token prompt through the "
    "decoder group (Full with per-query pools, 4 Reindex, 15 Reuse), windows cut to the replayed segment",
)

# Smaller cases of the same shapes, for parity at sizes the oracle finishes in seconds.
SMALL = {
    "tiny_bf16": replace(WORKLOADS["tiny_encoder"], name="tiny_bf16", act="bf16", kv="bf16"),
    "tiny_fp4": replace(WORKLOADS["tiny_encoder"], name="tiny_fp4", act="bf16", kv="fp4"),
    "decode_small": replace(WORKLOADS["decode_32k"], name="decode_small", batch=3, prior=3000, new=1),
    "decode_dense": replace(WORKLOADS["decode_32k"], name="decode_dense", batch=2, prior=400, new=1),
    "hsi_small": replace(
        WORKLOADS["decode_32k"], name="hsi_small", batch=2, prior=9000, new=1, topk=128, cand_blocks=64,
        layers=(LayerPlan("full", make_pool=True), LayerPlan("reindex", 0), LayerPlan("reuse", 1)),
    ),
    "group_small": replace(WORKLOADS["group_256k"], name="group_small", batch=2, prior=20000, new=1),
    "fp4_small": replace(WORKLOADS["fp4_1m"], name="fp4_small", batch=2, prior=20000, new=1),
    "fp4_pages": replace(WORKLOADS["fp4_1m"], name="fp4_pages", batch=2, prior=5000, new=1, main_group=16),
    # a pool level of 8752 block keys: the sampled first pass of the selection
    "pool_mid": replace(WORKLOADS["fp4_1m"], name="pool_mid", batch=1, prior=70000, new=1),
    "prefill_small": replace(WORKLOADS["prefill_128k"], name="prefill_small", prior=4096, new=512, n_q=512),
    "prefill_fp4_small": replace(WORKLOADS["prefill_128k"], name="prefill_fp4_small", kv="fp4", prior=4096, new=512,
                                 n_q=512),
    "multi_q_small": replace(WORKLOADS["decode_32k"], name="multi_q_small", batch=2, prior=2990, new=10, n_q=10),
    "encoder_block_small": replace(WORKLOADS["prefill_128k"], name="encoder_block_small", prior=4096, new=512,
                                   n_q=512, layers=ENCODER_BLOCK),
    # YaRN rotary extension (original length 65536, factor 16; theta 160000)
    "tiny_yarn": replace(WORKLOADS["tiny_encoder"], name="tiny_yarn", rope_factor=4.0, rope_orig_len=256),
    "decode_yarn": replace(WORKLOADS["decode_32k"], name="decode_yarn", batch=2, prior=5000, new=1,
                           rope_theta=160000.0, rope_factor=16.0, rope_orig_len=65536),
    "prefill_yarn": replace(WORKLOADS["prefill_128k"], name="prefill_yarn", prior=4096, new=512, n_q=512,
                            rope_theta=160000.0, rope_factor=16.0, rope_orig_len=65536),
    # a top-1536 (from a pool of 2048, and flat): the selection's threshold
    # level expands more than a thousand candidate blocks
    "pool_wide": replace(
        WORKLOADS["decode_32k"], name="pool_wide", batch=1, prior=20000, new=1, topk=1536,
        layers=(LayerPlan("full", make_pool=True), LayerPlan("reindex", 0), LayerPlan("reuse", 1)),
    ),
    "topk_wide": replace(WORKLOADS["decode_32k"], name="topk_wide", batch=1, prior=16000, new=1, topk=1536),
    # bounded replay: 128 queries whose windows stop at the segment start, the decoder group's modes
    "replay_small": replace(WORKLOADS["replay_64k"], name="replay_small", prior=6000 - 128, cand_blocks=64,
                            topk=128, layers=(LayerPlan("full", make_pool=True), LayerPlan("reuse", 0),
                                              LayerPlan("reindex", 0), LayerPlan("reuse", 2))),
    "decoder_prefill_small": replace(WORKLOADS["decoder_prefill_64k"], name="decoder_prefill_small", prior=8192,
                                     new=256, n_q=256, cand_blocks=64, topk=128),
    # FP8 (E4M3) window rows on every attention path: float32 generic, bf16
    # and FP4 caches, per-head-group and one-workgroup-per-query kernels
    "tiny_fp8win": replace(WORKLOADS["tiny_encoder"], name="tiny_fp8win", swa="fp8"),
    "decode_fp8win": replace(WORKLOADS["decode_32k"], name="decode_fp8win", batch=3, prior=3000, new=1, swa="fp8"),
    "fp4_pages_fp8win": replace(WORKLOADS["fp4_1m_pages"], name="fp4_pages_fp8win", prior=5000, new=1),
    "prefill_fp8win": replace(WORKLOADS["prefill_128k"], name="prefill_fp8win", prior=4096, new=512, n_q=512,
                              swa="fp8"),
    "prefill_fp4_fp8win": replace(WORKLOADS["prefill_128k"], name="prefill_fp4_fp8win", kv="fp4", prior=4096,
                                  new=512, n_q=512, swa="fp8"),
    # small chunks: 64 queries (a workgroup per head group), 128-255 queries
    # (a workgroup per query; bf16 rows with row splits, FP4 rows without)
    "chunk_small": replace(WORKLOADS["prefill_128k"], name="chunk_small", prior=4096, new=64, n_q=64),
    "chunk_fp4_small": replace(WORKLOADS["prefill_128k"], name="chunk_fp4_small", kv="fp4", prior=4096, new=200,
                               n_q=200),
    "chunk_fp8win": replace(WORKLOADS["prefill_128k"], name="chunk_fp8win", prior=4096, new=160, n_q=160,
                            swa="fp8"),
    # one query over a ratio-2 cache whose step writes one entry (two new
    # positions merged with the per-channel weights)
    "decode_r2_small": replace(WORKLOADS["decode_32k"], name="decode_r2_small", batch=3, ratio=2, prior=6000, new=2),
    "fp4_r2_small": replace(WORKLOADS["fp4_1m"], name="fp4_r2_small", batch=2, ratio=2, prior=10000, new=2),
}

ALL = {**WORKLOADS, **SMALL}


def _key(*parts) -> list:
    out = []
    for p in parts:
        out.append(zlib.crc32(p.encode()) if isinstance(p, str) else int(p))
    return out


def round_act(x: np.ndarray, act: str) -> np.ndarray:
    """float32 array whose values are representable in the activation dtype.

    bf16: round to nearest even on the float32 bit pattern (inputs only).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if act == "f32":
        return x
    if act != "bf16":
        raise ValueError(act)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


class Inputs:
    """All synthetic tensors of one workload (float32 arrays, values exact in the act dtype)."""

    def __init__(self, wl: Workload, seed: int = 0):
        self.wl = wl
        self.seed = seed

    def _rng(self, *parts) -> np.random.Generator:
        ss = np.random.SeedSequence(_key(self.seed, self.wl.name, *parts))
        return np.random.Generator(np.random.PCG64(ss))

    def _normal(self, shape, std, *parts) -> np.ndarray:
        x = self._rng(*parts).standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return x

    # ---- cache-side tensors -------------------------------------------------
    def latent(self, b: int, start: int, stop: int) -> np.ndarray:
        """Latent rows of sequence b at positions start .. stop-1, [stop-start, d]."""
        d = self.wl.d
        out = np.empty((max(0, stop - start), d), dtype=np.float32)
        c0, c1 = start // CHUNK, (stop - 1) // CHUNK if stop > start else start // CHUNK - 1
        for c in range(c0, c1 + 1):
            chunk = round_act(self._normal((CHUNK, d), 1.0, "latent", b, c), self.wl.act)
            lo, hi = max(start, c * CHUNK), min(stop, (c + 1) * CHUNK)
            out[lo - start : hi - start] = chunk[lo - c * CHUNK : hi - c * CHUNK]
        return out

    def pair_logits(self) -> np.ndarray | None:
        if self.wl.ratio == 1:
            return None
        return self._normal((self.wl.ratio, self.wl.d), 1.0, "pair_logits")

    def w_ik(self) -> np.ndarray:
        wl = self.wl
        return round_act(self._normal((wl.d, wl.d_idx), 1.0 / np.sqrt(wl.d), "w_ik"), wl.act)

    # ---- per-layer query-side tensors ----------------------------------------
    def q(self, layer: int) -> np.ndarray:
        wl = self.wl
        return round_act(self._normal((wl.batch, wl.n_q, wl.n_heads, wl.d), 1.0, "q", layer), wl.act)

    def q_idx(self, layer: int) -> np.ndarray:
        wl = self.wl
        return round_act(self._normal((wl.batch, wl.n_q, wl.n_idx_heads, wl.d_idx), 1.0, "q_idx", layer), wl.act)

    def head_w(self, layer: int) -> np.ndarray:
        wl = self.wl
        return self._normal((wl.batch, wl.n_q, wl.n_idx_heads), 1.0, "head_w", layer)

    def swa(self, layer: int) -> tuple[np.ndarray, np.ndarray]:
        """Window rows and the position of row 0 per sequence.

        FP8 windows are drawn directly as E4M3 (FN) code bytes: a random sign
        and a magnitude code uniform over 0x20 .. 0x3F (0.125 .. 1.875, unit
        scale like the N(0,1) rows), so the generator does no format
        arithmetic; each side decodes the bytes.
        """
        wl = self.wl
        first, n = wl.swa_span()
        firsts = np.full(wl.batch, first, dtype=np.int32)
        if wl.swa == "fp8":
            rng = self._rng("swa", layer)
            mag = rng.integers(0x20, 0x40, size=(wl.batch, n, wl.d), dtype=np.uint8)
            sign = rng.integers(0, 2, size=(wl.batch, n, wl.d), dtype=np.uint8) << 7
            return (mag | sign).astype(np.uint8), firsts
        rows = round_act(self._normal((wl.batch, n, wl.d), 1.0, "swa", layer), wl.act)
        return rows, firsts


def oproj_inputs(n_tok: int, width: int, n_groups: int, rank: int, act: str, seed: int = 0):
    """Seeded inputs of the grouped output projection: attention-output rows
    x [n_tok, width] (each channel a convex mix of unit-variance latent
    values: N(0, 0.25)) and group weights w [n_groups, rank, width/n_groups]
    with std 1/sqrt(K), both exact in the activation type."""
    k = width // n_groups
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(_key(seed, "oproj", n_tok, width, n_groups, rank))))
    x = rng.standard_normal((n_tok, width), dtype=np.float32) * np.float32(0.5)
    w = rng.standard_normal((n_groups, rank, k), dtype=np.float32) * np.float32(1.0 / np.sqrt(k))
    x, w = round_act(x, act), round_act(w, act)
    return x, w


def get(name: str) -> Workload:
    return ALL[name]
