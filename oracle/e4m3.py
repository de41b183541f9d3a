"""OCP 8-bit float E4M3 ("FN" variant) codec, by brute force -- test oracle.

Test infrastructure only (see the package docstring).

The pages name the cache type only as FP8 "F8E4M3" and say it roughly halves
the cache relative to FP16 ("PagedAttention in mistral.rs", section "KV Cache
Quantization").  Everything below that sentence is a reading:

* Format: sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinities; the
  only NaN magnitude is exponent 1111 with mantissa 111; largest finite
  magnitude 448; subnormals m * 2^-9.
* Encode: t = fp32(x) / fp32(scale) with IEEE fp32 division; NaN -> 0x7F with
  t's sign; |t| >= 448 (inf included) saturates to 0x7E with t's sign;
  otherwise the nearest finite magnitude, ties to the code whose last bit is 0
  (round to nearest even); the sign bit is t's sign bit, so -0 and tiny
  negatives become 0x80.
* Decode: the table value, times the scale, in fp64.

The encoder is written as the definition "pick the nearest representable
magnitude" over the full table, not as bit manipulation, so that it can be
checked by eye.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F
MAX_CODE = 0x7E


def code_value(code: int) -> float:
    """Value of one E4M3 code, straight from the format definition."""
    if not 0 <= code <= 0xFF:
        raise ValueError("code out of range")
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def table() -> np.ndarray:
    """All 256 code values as fp64 (NaN at 0x7F and 0xFF)."""
    return np.array([code_value(c) for c in range(256)], dtype=np.float64)


_TABLE = table()
# Codes 0x00..0x7E are the finite non-negative magnitudes, strictly increasing.
_MAGS = _TABLE[: MAX_CODE + 1].copy()
assert np.all(np.diff(_MAGS) > 0)


def quotient_f32(x, scale) -> np.ndarray:
    """t = fp32(x) / fp32(scale) with IEEE single-precision division."""
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.float32(scale)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (x32 / s32).astype(np.float32)


def encode_t(t) -> np.ndarray:
    """Encode already-divided fp32 values t to E4M3 codes (uint8)."""
    t = np.asarray(t, dtype=np.float32)
    flat = t.reshape(-1)
    sign = (flat.view(np.uint32) >> 31).astype(np.uint8) << 7
    a = np.abs(flat.astype(np.float64))
    out = np.empty(flat.shape, dtype=np.uint8)

    nan = np.isnan(a)
    sat = (~nan) & (a >= E4M3_MAX)
    mid = ~(nan | sat)

    # Nearest magnitude: a lies in (mags[lo], mags[hi]] with hi = lo + 1.
    am = a[mid]
    hi = np.searchsorted(_MAGS, am, side="left")
    hi = np.clip(hi, 0, MAX_CODE)
    exact = _MAGS[hi] == am
    lo = np.maximum(hi - 1, 0)
    # Midpoint of two adjacent magnitudes is exact in fp64.
    midpoint = (_MAGS[lo] + _MAGS[hi]) * 0.5
    pick = np.where(am < midpoint, lo, hi)
    tie = am == midpoint
    # On a tie the even code (last bit 0) wins.
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(exact, hi, pick)

    out[mid] = pick.astype(np.uint8)
    out[sat] = MAX_CODE
    out[nan] = NAN_CODE
    out |= sign
    return out.reshape(t.shape)


def encode(x, scale) -> np.ndarray:
    """E4M3 codes of fp32(x)/fp32(scale): divide, then :func:`encode_t`."""
    return encode_t(quotient_f32(x, scale))


def decode(codes, scale=1.0) -> np.ndarray:
    """fp64 values of codes, times fp64(scale)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _TABLE[codes] * np.float64(np.float32(scale))
