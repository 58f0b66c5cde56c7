"""Pins of the oracle's storage formats against definitions, library conversions and brute force."""
import numpy as np
import pytest
import torch

from oracle import formats


def test_bf16_table_matches_torch_decode():
    codes = np.arange(65536, dtype=np.int64)
    ref = torch.from_numpy(codes.astype(np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = formats.bf16_table()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_bf16_encode_matches_torch_rne_on_float32_inputs():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties: a bf16 value plus half of its ulp, both signs
    base = formats.bf16_round(rng.standard_normal(5000))
    ulp = np.abs(base) * 2.0 ** -7
    ties = np.concatenate([base + ulp / 2 * np.sign(base), base - ulp / 4]).astype(np.float32)
    x = np.concatenate([x, ties, np.float32([0.0, -0.0, 1e-40, -3e-39, 2.0 ** -133])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = formats.bf16_encode(x.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_encode_from_float64_is_single_rounding():
    # A float64 just above a bf16 midpoint must round up even though the float32
    # nearest to it is the midpoint itself (a double rounding would tie to even).
    lo = 1.0
    mid = 1.0 + 2.0 ** -8  # midpoint of 1.0 and 1.0078125
    x = mid + 2.0 ** -40
    assert np.float32(x) == np.float32(mid)
    assert formats.bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert formats.bf16_round(np.array([mid]))[0] == lo  # exact tie -> even code


def test_e4m3_table_matches_torch_decode():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = formats.e4m3_table()
    finite = np.isfinite(ref)
    assert np.array_equal(ours[finite], ref[finite])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    v = np.abs(rng.standard_normal(100_000)) * np.exp(rng.uniform(-9, 6, 100_000))
    v = np.minimum(v, 440.0).astype(np.float32)
    mids = (formats.e4m3_table()[1:0x7E] + formats.e4m3_table()[2:0x7F]) / 2
    v = np.concatenate([v, mids.astype(np.float32), np.float32([0.0, 448.0])])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = formats.e4m3_encode_scaled(v.astype(np.float64), 1.0)
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_scales_exactly():
    assert formats.e4m3_encode_scaled(np.array([1e6]), 6.0)[0] == 0x7E
    # amax/6 exactly at the midpoint of 1.0 and 1.125 -> even code (1.0)
    assert formats.e4m3_decode(formats.e4m3_encode_scaled(np.array([6 * 1.0625]), 6.0))[0] == 1.0
    # a hair above the midpoint rounds up although amax/6 in float64 would tie
    x = 6 * 1.0625 * (1 + 2.0 ** -52)
    assert formats.e4m3_decode(formats.e4m3_encode_scaled(np.array([x]), 6.0))[0] == 1.125


def _e2m1_from_bits(code: int) -> float:
    """E2M1 value from its bit fields: 1 sign, 2 exponent (bias 1), 1 mantissa."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -mag if s else mag


def test_e2m1_table_from_bit_fields():
    assert np.array_equal(formats.e2m1_table(), np.array([_e2m1_from_bits(c) for c in range(16)]))


def _e2m1_brute(x: float, scale: float) -> int:
    """Nearest E2M1 magnitude to x/scale by argmin over all 8, ties to the even code."""
    mags = [abs(_e2m1_from_bits(c)) for c in range(8)]
    dist = [abs(abs(x) - m * scale) for m in mags]
    best = min(dist)
    cands = [c for c in range(8) if dist[c] == best]
    c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
    if abs(x) > 6 * scale:
        c = 7
    return c | (8 if (x < 0 and c != 0) else 0)


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(3)
    scale = 0.375
    x = rng.uniform(-8, 8, 4000) * scale
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * scale
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 7 * scale, -100.0]])
    ours = formats.e2m1_encode_scaled(x, scale)
    ref = np.array([_e2m1_brute(v, scale) for v in x])
    assert np.array_equal(ours, ref)


def test_fp4_dequant_exact_in_bf16():
    vals = formats.e2m1_table()[:, None] * formats.e4m3_table()[None, :0x7F]
    vals = vals[np.isfinite(vals)]
    assert np.array_equal(formats.bf16_round(vals), vals)


def test_fp4_round_trip_and_error_bound():
    rng = np.random.default_rng(4)
    group = 16
    # Rows built from exact FP4 values whose group amax is 6*scale decode exactly.
    scales = formats.e4m3_table()[rng.integers(0x10, 0x60, size=(64, 4))]
    codes = rng.integers(0, 16, size=(64, 4, group))
    codes[..., 0] = 7  # amax = 6 * scale
    x = (formats.e2m1_table()[codes] * scales[..., None]).reshape(64, 4 * group)
    packed, sc = formats.fp4_encode(x, group)
    assert np.array_equal(formats.fp4_decode(packed, sc, group), x)
    # Gaussian rows: error at most half the local E2M1 spacing times the scale.
    y = rng.standard_normal((256, 64))
    packed, sc = formats.fp4_encode(y, 32)
    deq = formats.fp4_decode(packed, sc, 32)
    s = np.repeat(formats.e4m3_decode(sc), 32, axis=-1)
    mag = np.abs(y) / s
    spacing = np.where(mag < 2, 0.5, np.where(mag < 4, 1.0, 2.0))
    assert np.all(np.abs(y - deq) <= spacing / 2 * s + 1e-12)
    assert packed.shape == (256, 32) and sc.shape == (256, 2)


def test_fp4_packing_and_zero_scale():
    x = np.zeros((1, 32))
    x[0, 0], x[0, 1] = 6.0, -0.5
    packed, sc = formats.fp4_encode(x, 32)
    assert formats.e4m3_decode(sc)[0, 0] == 1.0
    assert packed[0, 0] == (0x7 | (0x9 << 4))  # even channel low nibble; -0.5 = sign|1
    packed, sc = formats.fp4_encode(np.full((1, 32), 1e-4), 32)  # amax/6 below half the min subnormal
    assert sc[0, 0] == 0 and np.all(packed == 0)
    packed, sc = formats.fp4_encode(np.full((1, 32), -1e-30), 32)
    assert np.all(packed == 0)  # never a negative zero code


@pytest.mark.parametrize("fmt", ["f32", "bf16", "fp4"])
def test_store_returns_dequantised_values(fmt):
    x = np.random.default_rng(5).standard_normal((8, 64))
    val, raw = formats.store(x, fmt, 32)
    assert val.shape == x.shape
    assert np.max(np.abs(val - x)) < (1e-6 if fmt == "f32" else 1e-2 if fmt == "bf16" else 1.0)
