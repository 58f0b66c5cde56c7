"""The seeded input generators both sides read (synth/): the same seed gives
the same arrays, each tensor, layer and sequence draws from its own stream,
latent rows read over any range (across the 4096-row generation chunks)
agree with one another, and the values are exactly representable in the
activation type.
"""
import numpy as np
import torch

import synth


def test_same_seed_same_arrays():
    wl = synth.get("hsi_small")
    a, b = synth.Inputs(wl), synth.Inputs(wl)
    assert np.array_equal(a.latent(1, 0, 300), b.latent(1, 0, 300))
    for layer in range(len(wl.layers)):
        assert np.array_equal(a.q(layer), b.q(layer))
        assert np.array_equal(a.q_idx(layer), b.q_idx(layer))
        assert np.array_equal(a.head_w(layer), b.head_w(layer))
        assert np.array_equal(a.swa(layer)[0], b.swa(layer)[0])
    assert np.array_equal(a.w_ik(), b.w_ik())
    # another seed draws other values
    assert not np.array_equal(a.q(0), synth.Inputs(wl, seed=1).q(0))


def test_streams_are_independent():
    wl = synth.get("hsi_small")
    inp = synth.Inputs(wl)
    assert not np.array_equal(inp.q(0), inp.q(1))
    assert not np.array_equal(inp.latent(0, 0, 64), inp.latent(1, 0, 64))
    assert not np.array_equal(inp.q_idx(0)[0, 0], inp.q_idx(0)[1, 0])
    # a workload's name keys its streams
    other = synth.Inputs(synth.get("decode_small"))
    assert not np.array_equal(inp.latent(0, 0, 64), other.latent(0, 0, 64))


def test_latent_ranges_agree_across_generation_chunks():
    wl = synth.get("decode_small")
    inp = synth.Inputs(wl)
    C = synth.CHUNK
    whole = inp.latent(2, 0, 2 * C + 17)
    assert whole.shape == (2 * C + 17, wl.d)
    for lo, hi in ((0, 1), (C - 3, C + 5), (C, C + 1), (C - 1, 2 * C + 17), (2 * C, 2 * C + 17), (5, 5)):
        assert np.array_equal(inp.latent(2, lo, hi), whole[lo:hi]), (lo, hi)


def test_values_are_exact_in_the_activation_type():
    inp = synth.Inputs(synth.get("decode_small"))
    for x in (inp.latent(0, 0, 100), inp.q(0), inp.q_idx(0), inp.w_ik(), inp.swa(0)[0]):
        assert x.dtype == np.float32
        assert np.all((x.view(np.uint32) & 0xFFFF) == 0)  # bf16 bit patterns
    tiny = synth.Inputs(synth.get("tiny_encoder"))  # float32 activations: no rounding
    assert np.any((tiny.q(0).view(np.uint32) & 0xFFFF) != 0)


def test_round_act_is_round_to_nearest_even():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(10000).astype(np.float32) * np.float32(1e3)
    # exact ties: a bf16 value plus half its last place, with odd and even last bits
    base = np.array([1.0, 1.0078125, 3.0, -2.015625], dtype=np.float32)
    ties = (base.view(np.uint32) + np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.round_act(x, "bf16"), want)
    assert np.array_equal(synth.round_act(x, "f32"), x)


def test_fp8_window_bytes_stay_in_their_code_range():
    wl = next(w for w in synth.SMALL.values() if w.swa == "fp8")
    rows, firsts = synth.Inputs(wl).swa(0)
    assert rows.dtype == np.uint8
    mag = rows & 0x7F
    assert mag.min() >= 0x20 and mag.max() <= 0x3F  # 0.125 .. 1.875 as E4M3 (FN)
    signs = rows >> 7
    assert 0.4 < signs.mean() < 0.6
    first, n = wl.swa_span()
    assert rows.shape == (wl.batch, n, wl.d) and np.all(firsts == first)
