"""Pins of the oracle's CSA2 steps against closed forms, brute force, library routines and invariants."""
import itertools
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle import csa2, driver, footprint, formats

import synth
from dataclasses import replace

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.strip() and not line.startswith("#"):
            key, rest = line.split(None, 1)
            out[key] = int(rest.split("|")[0])
    return out


# ---------------------------------------------------------------- footprint --


def test_footprint_matches_pages():
    g = _golden("footprint.txt")
    assert formats.fp4_entry_bytes(512, 16) == g["main_entry_bytes"]
    assert formats.fp4_entry_bytes(128, 32) == g["idx_entry_bytes"]
    main, idx = g["main_entry_bytes"], g["idx_entry_bytes"]
    assert 3 * Fraction(main, 2) == g["encoder_main_per_token"]
    assert 3 * Fraction(idx, 2) == g["encoder_idx_per_token"]
    assert footprint.bytes_per_token() == g["total_per_token"]
    # Only the mixed grouping (16 for main KV, 32 for indexer K) gives the pages' total.
    assert footprint.bytes_per_token(main_group=32) == 850
    assert footprint.bytes_per_token(idx_group=16) == 900
    # Chain from the previous generation's 584-byte FP8 main entry.
    v4_sources_4to1 = ((2, 4), (8, 4), (14, 4), (20, 4))
    assert footprint.chain_from_entry(584, 68, v4_sources_4to1) == g["chain_cross_layer"]
    assert footprint.chain_from_entry(584, 68, footprint.KV_SOURCES) == g["chain_ratio_relax"]
    assert round(g["v1_bytes_per_token"] / g["total_per_token"]) == g["v1_gap"]
    assert g["pool_blocks"] * g["pool_block_size"] == g["pool_positions"]


# --------------------------------------------------------------- compressor --


def test_compress_ratio1_is_identity():
    x = np.random.default_rng(0).standard_normal((10, 16))
    assert np.array_equal(csa2.compress(x, None, 1), x)


def test_compress_equal_logits_gives_mean_and_extremes_pick_one():
    rng = np.random.default_rng(1)
    # latent rows arrive in an activation type (float32 or bf16)
    x = rng.standard_normal((12, 8)).astype(np.float32).astype(np.float64)
    e = csa2.compress(x, np.zeros((2, 8)), 2)
    assert np.allclose(e, (x[0::2] + x[1::2]) / 2, rtol=0, atol=1e-15)
    logits = np.zeros((2, 8))
    logits[0, :4], logits[1, 4:] = 800.0, 800.0  # channel-wise: first half picks row 0, rest row 1
    e = csa2.compress(x, logits, 2)
    assert np.array_equal(e[:, :4], x[0::2, :4]) and np.array_equal(e[:, 4:], x[1::2, 4:])


def test_compress_of_equal_rows_is_that_row():
    # a convex combination of equal rows is the row itself, exactly, whatever
    # the weights: the stored code is then that of the row, ties included
    rng = np.random.default_rng(3)
    row = rng.standard_normal((5, 16)).astype(np.float32).astype(np.float64)
    x = np.repeat(row, 2, axis=0)
    for logits in (rng.standard_normal((2, 16)), np.zeros((2, 16)), 30 * rng.standard_normal((2, 16))):
        assert np.array_equal(csa2.compress(x, logits, 2), row)


def test_pair_weights_are_a_softmax_per_channel():
    a = np.random.default_rng(2).standard_normal((2, 32))
    w = csa2.pair_weights(a)
    assert np.allclose(w.sum(axis=0), 1.0, atol=1e-15)
    ref = torch.softmax(torch.from_numpy(a), dim=0).numpy()
    assert np.allclose(w, ref, atol=1e-15)


def test_entry_positions_and_visibility():
    assert list(csa2.entry_position(np.arange(3), 2)) == [1, 3, 5]
    # ratio 2: query 1008 sees entries 0..503 (entry 504 covers 1008,1009)
    assert csa2.visible_entries(512, 1008, 2) == 504
    assert csa2.visible_entries(512, 1009, 2) == 505
    assert csa2.visible_entries(512, 0, 2) == 0
    assert csa2.visible_entries(100, 5000, 1) == 100
    brute = lambda n, t, r: sum(1 for j in range(n) if r * j + r - 1 <= t)
    for n, t, r in itertools.product([0, 5, 17], range(-1, 40), [1, 2, 3]):
        assert csa2.visible_entries(n, t, r) == brute(n, t, r)


# --------------------------------------------------------------------- RoPE --


def test_rope_preserves_norm_and_leaves_nope_channels():
    x = np.random.default_rng(3).standard_normal((5, 64))
    y = csa2.rope(x, np.arange(5) * 1000 + 7, 16, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.array_equal(y[:, :48], x[:, :48])


def test_rope_matches_complex_rotation_and_is_relative():
    rng = np.random.default_rng(4)
    d, dr, theta = 32, 16, 10000.0
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    t = 777
    z = (q[d - dr :: 2] + 1j * q[d - dr + 1 :: 2]) * np.exp(1j * t * theta ** (-np.arange(dr // 2) * 2.0 / dr))
    y = csa2.rope(q, t, dr, theta)
    assert np.allclose(y[d - dr :: 2], z.real, atol=1e-12) and np.allclose(y[d - dr + 1 :: 2], z.imag, atol=1e-12)
    # q.k after rotation depends only on the offset t - p
    a = csa2.rope(q, 1000, dr, theta) @ csa2.rope(k, 900, dr, theta)
    b = csa2.rope(q, 123456, dr, theta) @ csa2.rope(k, 123356, dr, theta)
    assert abs(a - b) < 1e-9


def test_rope_frequencies_hand_worked():
    """Rotation angles worked by hand for theta = 10000: with 4 rotary
    channels pair 0 turns 1 rad per position and pair 1 turns
    10000^(-1/2) = 0.01 rad, so at position 100 the pairs have turned 100 rad
    and exactly 1 rad; with 8 rotary channels pair 2 turns 10000^(-1/2) too."""
    x = np.array([5.0, 1.0, 0.0, 1.0, 0.0])  # one non-rotary channel, then pairs (1, 0), (1, 0)
    y = csa2.rope(x, 100, 4, 10000.0)
    assert y[0] == 5.0
    assert np.allclose(y[1:3], [np.cos(100.0), np.sin(100.0)], atol=1e-12)
    assert np.allclose(y[3:5], [np.cos(1.0), np.sin(1.0)], atol=1e-12)
    z = csa2.rope(np.array([1.0, 0.0] * 4), 100, 8, 10000.0)
    assert np.allclose(z[4:6], [np.cos(1.0), np.sin(1.0)], atol=1e-12)
    assert np.allclose(z[2:4], [np.cos(10.0), np.sin(10.0)], atol=1e-12)  # 10000^(-1/4) = 0.1 rad per position


# ------------------------------------------------------------------- scores --


def test_indexer_score_invariants():
    """The score formula itself is a reading (parity unpinned); these are its invariants."""
    rng = np.random.default_rng(5)
    q, w, K = rng.standard_normal((4, 16)), rng.standard_normal(4), rng.standard_normal((50, 16))
    s = csa2.indexer_scores(q, w, K)
    assert np.allclose(csa2.indexer_scores(3.0 * q, w, K), 3.0 * s)  # positive homogeneity in q
    assert np.allclose(csa2.indexer_scores(q, 2.0 * w, K), 2.0 * s)  # linear in w
    assert np.all(csa2.indexer_scores(q, np.abs(w), K) >= 0)
    # one head, unit weight: plain ReLU of a dot product (library matvec)
    one = csa2.indexer_scores(q[:1], np.ones(1), K)
    assert np.allclose(one, torch.relu(torch.from_numpy(K) @ torch.from_numpy(q[0])).numpy())
    # negated query on every head: scores of heads with all-negative dots vanish
    assert np.all(csa2.indexer_scores(-np.abs(q), np.ones(4), np.abs(K)) == 0)


def test_indexer_score_relu_is_per_head_hand_worked():
    """Two heads whose dot products have opposite signs separate a ReLU taken
    per head from one taken after the weighted head sum (the reading of the
    zartbot walkthrough, 2.3.1: each head's score is clipped at zero before
    the query's head weights combine them).  Values worked by hand."""
    K = np.array([[1.0, 0.0], [0.0, 1.0]])  # entry 0 = e0, entry 1 = e1
    q = np.array([[2.0, 0.0], [-3.0, 0.0]])  # head 0 . e0 = +2, head 1 . e0 = -3; both 0 on e1
    # w = (1, 1): per head 1*2 + 1*0 = 2 (after the sum it would be max(0, -1) = 0)
    assert list(csa2.indexer_scores(q, np.array([1.0, 1.0]), K)) == [2.0, 0.0]
    # w = (1, -1): the negative weight meets a clipped head, so it adds nothing:
    # 1*2 + (-1)*0 = 2 (after the sum: max(0, 2 + 3) = 5)
    assert list(csa2.indexer_scores(q, np.array([1.0, -1.0]), K)) == [2.0, 0.0]
    # w = (-1, 1): a negative weight on the positive head makes the score negative,
    # -2 + 0 = -2 (after the sum it could never fall below 0)
    assert list(csa2.indexer_scores(q, np.array([-1.0, 1.0]), K)) == [-2.0, 0.0]
    # three heads, integer arithmetic: dots (4, -1, 3), w (0.5, 7, -2) -> 2 + 0 - 6 = -4
    q3 = np.array([[4.0, 0.0], [-1.0, 0.0], [3.0, 0.0]])
    assert csa2.indexer_scores(q3, np.array([0.5, 7.0, -2.0]), K[:1])[0] == -4.0


# -------------------------------------------------------------------- top-k --


def _brute_topk(scores, ids, k):
    pairs = sorted(zip(scores.tolist(), ids.tolist()), key=lambda p: (-p[0], p[1]))[:k]
    out = sorted(i for _, i in pairs)
    return out + [-1] * (k - len(out))


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(6)
    for trial in range(300):
        n = int(rng.integers(0, 60))
        s = rng.integers(-5, 5, n).astype(np.float64)  # heavy ties
        ids = np.sort(rng.choice(1000, n, replace=False))
        k = int(rng.integers(1, 40))
        assert list(csa2.topk_select(s, ids, k)) == _brute_topk(s, ids, k)


def test_hsi_pool_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(200):
        beta, kappa = int(rng.integers(1, 5)), int(rng.integers(1, 8))
        n = int(rng.integers(1, 50))
        s = rng.integers(0, 6, n).astype(np.float64)
        pool = csa2.hsi_pool(s, beta, kappa)
        nb = -(-n // beta)
        bmax = [max(s[b * beta : (b + 1) * beta]) for b in range(nb)]
        if nb <= kappa:
            exp = list(range(nb))
        else:
            forced = (n - 1) // beta
            rest = sorted((b for b in range(nb) if b != forced), key=lambda b: (-bmax[b], b))[: kappa - 1]
            exp = sorted([forced] + rest)
        assert list(pool) == exp + [-1] * (kappa - len(exp))
        chosen = set(b for b in pool if b >= 0)
        assert (n - 1) // beta in chosen and len(chosen) == min(kappa, nb)


def test_hierarchical_equals_flat_when_pool_exceeds_k():
    """Top-k within the HSI pool equals the flat top-k whenever kappa - 1 >= k."""
    rng = np.random.default_rng(8)
    for trial in range(300):
        beta = int(rng.integers(1, 9))
        k = int(rng.integers(1, 12))
        kappa = k + 1 + int(rng.integers(0, 4))
        n = int(rng.integers(1, 200))
        s = np.round(rng.standard_normal(n), 1)  # ties present
        pool = csa2.hsi_pool(s, beta, kappa)
        dom = csa2.pool_domain(pool, beta, n)
        assert list(csa2.topk_select(s[dom], dom, k)) == list(csa2.topk_select(s, np.arange(n), k))


# ---------------------------------------------------------------- attention --


def test_attention_matches_torch_sdpa_and_invariants():
    rng = np.random.default_rng(9)
    H, d, dr, n, t = 4, 32, 8, 37, 500
    q, rows = rng.standard_normal((H, d)), rng.standard_normal((n, d))
    out, p, lse = csa2.attention(q, t, rows, dr, 10000.0)
    qh = torch.from_numpy(csa2.rope(q, t, dr, 10000.0))[None, :, None, :]  # [1, H, 1, d]
    kv = torch.from_numpy(rows)[None, None].expand(1, H, n, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kv, kv)[0, :, 0].numpy()
    assert np.allclose(out, ref, atol=1e-12)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
    logits = csa2.rope(q, t, dr, 10000.0) @ rows.T / np.sqrt(d)
    assert np.allclose(lse, logsumexp(logits, axis=1), atol=1e-12)
    # convex hull: every output channel lies within the rows' range
    assert np.all(out <= rows.max(axis=0) + 1e-12) and np.all(out >= rows.min(axis=0) - 1e-12)


def test_dense_when_topk_covers_everything():
    """k >= entries: the sparse step reduces to dense causal attention over all visible entries + window."""
    wl = synth.get("decode_dense")
    inp = synth.Inputs(wl)
    res, caches = driver.run_step(inp)
    for b in range(wl.batch):
        t = int(wl.q_positions()[b, 0])
        n_vis = csa2.visible_entries(caches[b].n_entries, t, wl.ratio)
        assert list(res[0]["topk"][b, 0][:n_vis]) == list(range(n_vis))
        swa, first = inp.swa(0)
        win = swa[b].astype(np.float64)[max(0, t - wl.window + 1) - first[b] :]
        rows = np.concatenate([caches[b].main_rows(np.arange(n_vis)), win])
        q = torch.from_numpy(csa2.rope(inp.q(0)[b, 0].astype(np.float64), t, wl.d_rope, wl.rope_theta))
        kv = torch.from_numpy(rows)
        ref = torch.softmax(q @ kv.T / np.sqrt(wl.d), dim=-1) @ kv
        assert np.allclose(res[0]["out"][b, 0], ref.numpy(), atol=1e-12)


def test_window_rows_clip_to_buffer_and_sequence_start():
    assert list(csa2.window_positions(3, 16)) == [0, 1, 2, 3]
    assert len(csa2.window_positions(1000, 128)) == 128


# -------------------------------------------------------------------- group --


def test_group_mode_invariants():
    wl = synth.get("hsi_small")  # Full(pool) -> Reindex(pool) -> Reuse(Reindex)
    inp = synth.Inputs(wl)
    res, caches = driver.run_step(inp)
    full, reidx, reuse = res
    assert np.array_equal(reuse["topk"], reidx["topk"])  # Reuse: bit-identical indices
    for b in range(wl.batch):
        pool = full["pool"][b, 0]
        t = int(wl.q_positions()[b, 0])
        n_vis = csa2.visible_entries(caches[b].n_entries, t, wl.ratio)
        assert (n_vis - 1) // wl.block_size in set(pool)
        # every Reindex pick lies inside the pool
        picks = reidx["topk"][b, 0]
        assert set(p // wl.block_size for p in picks if p >= 0) <= set(pool)


def test_reindex_with_full_query_reproduces_full():
    wl = synth.get("hsi_small")
    inp = synth.Inputs(wl)
    dims = driver.dims_of(wl)
    cache = driver.build_cache(inp, 0, wl.context)
    t = wl.context - 1
    qi, w = inp.q_idx(0)[0, 0].astype(np.float64), inp.head_w(0)[0, 0].astype(np.float64)
    top, pool, _ = csa2.full_query(dims, cache, cache.n_entries, t, qi, w, True)
    flat, _, _ = csa2.reindex_query(dims, cache, cache.n_entries, t, qi, w, None)
    assert np.array_equal(top, flat)
    big = driver.dims_of(wl)
    big.cand_blocks = wl.topk + 1  # kappa - 1 >= k: pool search equals flat
    _, pool2, _ = csa2.full_query(big, cache, cache.n_entries, t, qi, w, True)
    inpool, _, _ = csa2.reindex_query(big, cache, cache.n_entries, t, qi, w, pool2)
    assert np.array_equal(inpool, top)


def test_group_rejects_later_source():
    dims = csa2.Dims(d=8, d_rope=2, n_heads=1, n_idx_heads=1, d_idx=4, topk=2, window=2)
    with pytest.raises(ValueError):
        csa2.run_group(dims, [], [], np.zeros((0, 1), dtype=int), [csa2.LayerSpec("reuse", source=0)])


def test_cache_is_post_rope_and_index_k_from_unrounded_entry():
    wl = synth.get("tiny_encoder")
    inp = synth.Inputs(wl)
    x = inp.latent(0, 0, 64).astype(np.float64)
    main, _, idx, _, e_hat = csa2.make_entries(x, 0, inp.pair_logits(), inp.w_ik(), 2, 16, 10000.0, "f32")
    e = csa2.compress(x, inp.pair_logits(), 2)
    assert np.allclose(np.linalg.norm(e_hat, axis=1), np.linalg.norm(e, axis=1))
    assert np.array_equal(main, formats.f32_round(e_hat))
    assert np.array_equal(idx, formats.f32_round(e_hat @ inp.w_ik().astype(np.float64)))


# ---- YaRN rotary extension ([ZB] 1.2 names original length 65536, factor 16)

YARN = csa2.Rope(160000.0, 16.0, 65536)


def test_yarn_off_is_plain_rope():
    x = np.random.default_rng(11).standard_normal((3, 64))
    for off in (csa2.Rope(10000.0, 1.0, 65536), csa2.Rope(10000.0, 0.0, 0)):
        assert np.array_equal(csa2.rope_freqs(off, 16), csa2.rope_freqs(10000.0, 16))
        assert np.array_equal(csa2.rope(x, 77, 16, off), csa2.rope(x, 77, 16, 10000.0))
        assert csa2.logit_temperature(off) == 1.0


def test_yarn_keeps_short_wavelengths_and_stretches_long_ones():
    plain = csa2.rope_freqs(YARN.theta, 64)
    f = csa2.rope_freqs(YARN, 64)
    fits = YARN.orig_len * plain / (2 * np.pi)  # wavelengths inside the original context
    assert np.array_equal(f[fits >= 32], plain[fits >= 32])  # short wavelengths untouched
    assert np.allclose(f[fits <= 1], plain[fits <= 1] / YARN.factor, rtol=1e-15, atol=0)  # long: interpolated
    mid = (fits > 1) & (fits < 32)
    assert mid.any() and (fits >= 32).any() and (fits <= 1).any()  # all three regimes occur at d_rope 64
    assert np.all(f[mid] < plain[mid]) and np.all(f[mid] > plain[mid] / YARN.factor)
    assert np.all(np.diff(f) < 0)  # still strictly decreasing over the pairs
    # the wavelength of the longest interpolated pair grows by the factor: it spans
    # factor x the original context that the plain one spanned
    assert np.isclose(2 * np.pi / f[-1], YARN.factor * 2 * np.pi / plain[-1], rtol=1e-14)


def test_yarn_rotation_is_relative_and_norm_preserving():
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal((2, 128))
    a = csa2.rope(q, 900_000, 64, YARN) @ csa2.rope(k, 899_500, 64, YARN)
    b = csa2.rope(q, 1500, 64, YARN) @ csa2.rope(k, 1000, 64, YARN)
    assert np.isclose(a, b, rtol=1e-9, atol=1e-9)
    x = rng.standard_normal((4, 128))
    assert np.allclose(np.linalg.norm(csa2.rope(x, 1_000_000, 64, YARN), axis=1), np.linalg.norm(x, axis=1))


def test_yarn_temperature_grows_with_the_factor():
    ts = [csa2.logit_temperature(csa2.Rope(10000.0, s, 65536)) for s in (1.0, 2.0, 4.0, 16.0, 64.0)]
    assert ts[0] == 1.0 and all(b > a for a, b in zip(ts, ts[1:]))


# ------------------------------------------------------------ lazy cache --


def _lazy_matches_built(wl, ids):
    inp = synth.Inputs(wl)
    built = driver.build_cache(inp, 0, wl.context)
    lazy = driver.LazyMainCache(inp, 0, wl.context)
    assert lazy.n_entries == built.n_entries == wl.capacity
    for key, arr in built.idx_raw.items():  # the whole indexer K, byte for byte
        assert np.array_equal(lazy.idx_raw[key], arr), key
    ids = np.asarray(ids, dtype=np.int64)
    rows = lazy.main_raw_rows(ids)
    assert set(rows) == set(built.main_raw)
    for key, arr in built.main_raw.items():  # main-KV rows made on demand
        assert np.array_equal(rows[key], arr[ids]), key
    assert np.array_equal(lazy.main_rows(ids), built.main_rows(ids))


def test_lazy_main_cache_equals_built_cache_ratio2():
    """The deferred main-KV rows and the indexer K of LazyMainCache are the
    bytes build_cache stores, at ratio 2, on both sides of the 4096-position
    latent fetches (entries 2047/2048, 4095/4096) and of the 16384-position
    build chunks (entries 8191/8192), first and last entries included."""
    wl = replace(synth.get("tiny_encoder"), name="lazy_ratio2", prior=2 * 8300, new=0, n_q=1)
    _lazy_matches_built(wl, [0, 1, 2047, 2048, 2049, 4095, 4096, 8191, 8192, 8193, wl.capacity - 1, 5, 4096])


def test_lazy_main_cache_equals_built_cache_fp4_pages():
    """The same in the pages' FP4 format (main KV one E4M3 scale per 16
    channels, indexer K per 32) at ratio 1, across the 4096-entry fetch and
    the 16384-entry build chunk."""
    wl = replace(synth.get("fp4_pages"), name="lazy_fp4_pages", batch=1, prior=16400, new=1, n_q=1)
    _lazy_matches_built(wl, [0, 4095, 4096, 8191, 8192, 12288, 16383, 16384, 16385, wl.capacity - 1])
