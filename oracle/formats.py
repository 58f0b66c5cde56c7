"""Storage number formats of the CSA2 cache, written from their definitions.

TEST INFRASTRUCTURE ONLY.  This package is the oracle: a plain, slow CPU
statement of what the CSA2 path computes.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
does.

Formats (each table is built by enumerating every code of the format):

* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits.
* E4M3 ("FN" variant of the OCP 8-bit float spec): 1 sign, 4 exponent
  (bias 7), 3 mantissa bits, subnormals, no infinities, code 0x7F/0xFF = NaN,
  largest finite 448.
* E2M1 (OCP 4-bit float): magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in
  bit 3.

Rounding is always "nearest representable value, ties to the even code",
found by searching the enumerated table.  Every comparison is made exact:
the decision between two neighbours a < b is taken by comparing the input
with (a + b) / 2, which is exactly representable in float64 for every pair
of neighbours in these tables.

The FP4 block codec follows the pages' description of the FP4 main-KV cache
(zartbot walkthrough, hn.213312.xyz, section 2.4.4; 36Kr "What black
technologies does DeepSeek V4.1 Flash adopt?", heading "FP4 and Bounded
Replay"): E2M1 elements sharing one E4M3 scale per group of channels.  The
pages state the group as 16 channels for the main KV and imply 32 for the
indexer K through its 68-byte entry (walkthrough section 3.1); the group is a
parameter here.  Readings taken where the pages are silent:

* scale = E4M3 value nearest to amax / 6 (ties to even), saturating at 448;
* a zero scale stores all-zero codes;
* element code = E2M1 value v nearest to x / scale (ties to the even code),
  saturating at +-6; a zero magnitude is stored as code 0 (never -0);
* packing: two codes per byte, the even channel in the low nibble;
* dequantised value = E2M1 value x scale.
"""
from __future__ import annotations

import numpy as np

# --------------------------------------------------------------------------
# Enumerated tables
# --------------------------------------------------------------------------


def bf16_table() -> np.ndarray:
    """float64 value of every bfloat16 bit pattern 0..65535 (NaN for NaN codes)."""
    codes = np.arange(65536, dtype=np.int64)
    sign = np.where((codes >> 15) & 1, -1.0, 1.0)
    exp = (codes >> 7) & 0xFF
    man = (codes & 0x7F).astype(np.float64)
    vals = np.where(
        exp == 0,
        man / 128.0 * 2.0 ** -126,
        (1.0 + man / 128.0) * np.power(2.0, (exp - 127).astype(np.float64)),
    )
    vals = np.where(exp == 0xFF, np.where(man == 0, np.inf, np.nan), vals)
    return sign * vals


def e4m3_table() -> np.ndarray:
    """float64 value of every E4M3 (FN) code 0..255 (NaN for 0x7F / 0xFF)."""
    codes = np.arange(256, dtype=np.int64)
    sign = np.where((codes >> 7) & 1, -1.0, 1.0)
    exp = (codes >> 3) & 0xF
    man = (codes & 0x7).astype(np.float64)
    vals = np.where(
        exp == 0,
        man / 8.0 * 2.0 ** -6,
        (1.0 + man / 8.0) * np.power(2.0, (exp - 7).astype(np.float64)),
    )
    vals = np.where((codes & 0x7F) == 0x7F, np.nan, vals)
    return sign * vals


E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_table() -> np.ndarray:
    """float64 value of every E2M1 code 0..15 (bit 3 is the sign)."""
    return np.concatenate([E2M1_MAGNITUDES, -E2M1_MAGNITUDES])


_BF16 = bf16_table()
_E4M3 = e4m3_table()
_E2M1 = e2m1_table()

# Non-negative finite values in code order (monotone increasing in the code).
_BF16_POS_CODES = np.arange(0, 0x7F81, dtype=np.int64)  # 0x0000 .. 0x7F80 (+inf last)
_BF16_POS_VALS = _BF16[_BF16_POS_CODES]
_E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)  # 0x00 .. 0x7E (448)
_E4M3_POS_VALS = _E4M3[_E4M3_POS_CODES]


def _nearest_even(target: np.ndarray, vals: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Code of the table value nearest to each non-negative ``target``.

    ``vals`` is increasing and ``codes`` gives each value's code.  Targets at
    or above the last value map to the last code (saturation).  A target at
    the exact midpoint of two neighbours takes the even code.
    """
    t = np.asarray(target, dtype=np.float64)
    hi = np.searchsorted(vals, t, side="left")  # vals[hi-1] < t <= vals[hi]
    hi = np.clip(hi, 1, len(vals) - 1)
    lo = hi - 1
    a, b = vals[lo], vals[hi]
    mid = (a + b) * 0.5  # exact for neighbours of every table used here
    pick_hi = (t > mid) | ((t == mid) & (codes[hi] % 2 == 0))
    out = np.where(pick_hi, codes[hi], codes[lo])
    out = np.where(t >= vals[-1], codes[-1], out)
    out = np.where(t <= vals[0], codes[0], out)
    return out


# --------------------------------------------------------------------------
# bfloat16 and float32 storage
# --------------------------------------------------------------------------


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """Round float64 ``x`` to the nearest bfloat16 (ties to even); uint16 codes.

    Finite inputs beyond the largest finite bfloat16 raise: the cache never
    holds such values.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_encode: non-finite input")
    mag = np.abs(x)
    if np.any(mag >= _BF16[0x7F7F]):
        raise ValueError("bf16_encode: input outside the finite bfloat16 range")
    code = _nearest_even(mag, _BF16_POS_VALS[:-1], _BF16_POS_CODES[:-1])
    sign = np.signbit(x).astype(np.int64) << 15
    return (code | sign).astype(np.uint16)


def bf16_decode(codes: np.ndarray) -> np.ndarray:
    return _BF16[np.asarray(codes, dtype=np.int64)]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 value of the bfloat16 nearest to ``x``."""
    return bf16_decode(bf16_encode(x))


def f32_round(x: np.ndarray) -> np.ndarray:
    """float64 value of the float32 nearest to ``x`` (numpy's IEEE conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# E4M3 and E2M1
# --------------------------------------------------------------------------


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.int64)]


def e4m3_encode_scaled(v: np.ndarray, k: float = 1.0) -> np.ndarray:
    """Code of the non-negative E4M3 value s nearest to ``v / k`` (ties to even).

    The search runs over the table k*s, so the division is never rounded; for
    k = 6 every k*s is exact in float64.  Saturates at 448 (code 0x7E).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0):
        raise ValueError("e4m3_encode_scaled: negative input")
    return _nearest_even(v, _E4M3_POS_VALS * k, _E4M3_POS_CODES).astype(np.uint8)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return _E2M1[np.asarray(codes, dtype=np.int64)]


def e2m1_encode_scaled(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E2M1 code of the value v with v*scale nearest to ``x`` (ties to even code).

    ``scale`` must be > 0 and broadcast against ``x``; magnitudes beyond 6*scale
    saturate to code 7.  A zero magnitude is code 0 whatever the sign of x.
    """
    x = np.asarray(x, dtype=np.float64)
    scale = np.broadcast_to(np.asarray(scale, dtype=np.float64), x.shape)
    mag = np.abs(x)
    mags = E2M1_MAGNITUDES
    code = np.zeros(x.shape, dtype=np.int64)
    # Walk the seven midpoints between consecutive magnitudes: the nearest
    # magnitude index is the number of midpoints below |x|, with a midpoint
    # equal to |x| counted only when the upper neighbour's code is even.
    for i in range(len(mags) - 1):
        mid = (mags[i] + mags[i + 1]) * 0.5 * scale  # exact: few significant bits
        upper_even = (i + 1) % 2 == 0
        code += (mag > mid) | ((mag == mid) & upper_even)
    sign = (np.signbit(x) & (code != 0)).astype(np.int64) << 3
    return (code | sign).astype(np.uint8)


# --------------------------------------------------------------------------
# FP4 block codec
# --------------------------------------------------------------------------


def fp4_encode(x: np.ndarray, group: int) -> tuple[np.ndarray, np.ndarray]:
    """Quantise rows ``x[..., ch]`` to FP4 with one E4M3 scale per ``group`` channels.

    Returns ``(packed, scales)``: packed uint8 ``[..., ch/2]`` (even channel in
    the low nibble) and uint8 E4M3 scale codes ``[..., ch/group]``.
    """
    x = np.asarray(x, dtype=np.float64)
    ch = x.shape[-1]
    if ch % group or ch % 2:
        raise ValueError("fp4_encode: channel count must be a multiple of the group and of 2")
    g = x.reshape(x.shape[:-1] + (ch // group, group))
    amax = np.abs(g).max(axis=-1)
    scale_codes = e4m3_encode_scaled(amax, 6.0)
    scale = e4m3_decode(scale_codes)
    safe = np.where(scale > 0, scale, 1.0)[..., None]
    codes = e2m1_encode_scaled(g, safe)
    codes = np.where((scale > 0)[..., None], codes, 0).astype(np.uint8)
    codes = codes.reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_codes


def fp4_decode(packed: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """float64 values of FP4 rows: E2M1 value times the group's E4M3 scale."""
    packed = np.asarray(packed, dtype=np.uint8)
    lo = packed & 0xF
    hi = packed >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(packed.shape[:-1] + (packed.shape[-1] * 2,))
    vals = e2m1_decode(codes)
    sc = e4m3_decode(scales)
    return vals * np.repeat(sc, group, axis=-1)


def fp4_entry_bytes(channels: int, group: int) -> int:
    """Bytes one FP4 row occupies: half a byte per element plus one scale byte per group.

    Counted from the codec's own output arrays, so the figure follows the
    format, not a formula typed a second time.
    """
    packed, scales = fp4_encode(np.zeros((1, channels)), group)
    return packed.shape[-1] * packed.itemsize + scales.shape[-1] * scales.itemsize


# --------------------------------------------------------------------------
# Generic storage
# --------------------------------------------------------------------------


def store(x: np.ndarray, fmt: str, group: int = 32) -> tuple[np.ndarray, dict]:
    """Round ``x`` to the storage format ``fmt``; return (dequantised float64, raw parts).

    fmt is "f32", "bf16" or "fp4".  Raw parts: {"f32": float32 array},
    {"bf16": uint16 codes} or {"codes": packed uint8, "scales": uint8}.
    """
    if fmt == "f32":
        raw = np.asarray(x, dtype=np.float64).astype(np.float32)
        return raw.astype(np.float64), {"f32": raw}
    if fmt == "bf16":
        codes = bf16_encode(x)
        return bf16_decode(codes), {"bf16": codes}
    if fmt == "fp4":
        packed, scales = fp4_encode(x, group)
        return fp4_decode(packed, scales, group), {"codes": packed, "scales": scales}
    raise ValueError(f"unknown storage format {fmt!r}")
