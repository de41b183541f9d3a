"""Pins for the oracle's E4M3 codec (CPU only).

The pages name the format only as F8E4M3 ("PagedAttention in mistral.rs",
section "KV Cache Quantization").  The pins below tie the oracle to the OCP
8-bit floating point definition (E4M3: bias 7, max 448, NaN = S.1111.111,
no infinities) through literal spot values, hand-worked ties, and an
independent implementation: torch's ``float8_e4m3fn`` cast, which agrees with
round-to-nearest-even for every |t| <= 464 (above that torch returns NaN
where the oracle saturates, by the saturation reading).
"""

import math

import numpy as np
import pytest
import torch

from oracle import e4m3

# Literal spot values of the E4M3 format (not computed from the oracle's formula).
SPOT = {
    0x00: 0.0,
    0x01: 2.0 ** -9,          # smallest subnormal
    0x07: 7 * 2.0 ** -9,      # largest subnormal
    0x08: 2.0 ** -6,          # smallest normal
    0x38: 1.0,
    0x39: 1.125,
    0x3A: 1.25,
    0x40: 2.0,
    0x77: 240.0,
    0x78: 256.0,
    0x7E: 448.0,              # largest finite
    0xB8: -1.0,
    0xFE: -448.0,
}


def test_spot_values():
    tab = e4m3.table()
    for code, val in SPOT.items():
        assert tab[code] == val, hex(code)
    assert math.isnan(tab[0x7F]) and math.isnan(tab[0xFF])
    assert tab[0x80] == 0.0 and math.copysign(1.0, tab[0x80]) == -1.0


def test_table_shape_facts():
    tab = e4m3.table()
    finite = tab[~np.isnan(tab)]
    assert finite.size == 254
    assert finite.max() == 448.0 and finite.min() == -448.0
    pos = np.unique(finite[finite > 0])
    assert pos.size == 126
    # Strictly increasing magnitudes over codes 0x00..0x7E.
    assert np.all(np.diff(tab[:0x7F]) > 0)


def test_round_trip_all_codes():
    tab = e4m3.table()
    codes = np.array([c for c in range(256) if not np.isnan(tab[c])], dtype=np.uint8)
    back = e4m3.encode_t(tab[codes].astype(np.float32))
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("t,code", [
    (1.0625, 0x38),            # tie 1.0 / 1.125 -> even 0x38
    (1.1875, 0x3A),            # tie 1.125 / 1.25 -> even 0x3A
    (2.0 ** -10, 0x00),        # tie 0 / 2^-9 -> even 0x00
    (3 * 2.0 ** -10, 0x02),    # tie 2^-9 / 2^-8 -> even 0x02
    (-(2.0 ** -11), 0x80),     # rounds to -0
    (-0.0, 0x80),
    (0.0, 0x00),
    (1.07, 0x39),              # just above the 1.0625 tie
    (1.06, 0x38),
    (464.0, 0x7E),
    (470.0, 0x7E),             # saturates
    (1e30, 0x7E),
    (float("inf"), 0x7E),
    (float("-inf"), 0xFE),
    (-500.0, 0xFE),
    (float("nan"), 0x7F),
    (232.0, 0x76),             # tie 224 / 240 -> even 0x76 (224)
    (248.0, 0x78),             # tie 240 / 256 -> even 0x78 (256)
])
def test_hand_worked_codes(t, code):
    assert int(e4m3.encode_t(np.float32(t))) == code


def _torch_codes(t32):
    return torch.from_numpy(t32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_matches_torch_cast_random():
    rng = np.random.default_rng(123)
    t = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 50,
        rng.uniform(-464, 464, 100_000).astype(np.float32),
        (rng.standard_normal(100_000) * 2.0 ** -8).astype(np.float32),
    ])
    assert np.array_equal(e4m3.encode_t(t), _torch_codes(t))


@pytest.mark.parametrize("scale", [1.0, 0.0107421875, 3.0, float(np.float32(4.7) / np.float32(448))])
def test_exhaustive_bf16_inputs_vs_torch(scale):
    """Every bf16 bit pattern, divided by an fp32 scale, against torch's cast."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    t = e4m3.quotient_f32(x, scale)
    ours = e4m3.encode_t(t)
    ok = np.isfinite(t) & (np.abs(t) <= 464)
    assert np.array_equal(ours[ok], _torch_codes(t[ok]))
    big = np.isfinite(t) & (np.abs(t) > 464)
    assert np.all((ours[big] & 0x7F) == 0x7E)
    nan = np.isnan(t)
    assert np.all((ours[nan] & 0x7F) == 0x7F)


def test_exhaustive_f16_inputs_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    for scale in (1.0, 0.25, 0.0107421875):
        t = e4m3.quotient_f32(x, scale)
        ours = e4m3.encode_t(t)
        ok = np.isfinite(t) & (np.abs(t) <= 464)
        assert np.array_equal(ours[ok], _torch_codes(t[ok]))


def test_division_is_ieee_f32():
    # 1/3 in fp32 differs from the fp64 quotient rounded once more; the oracle
    # must use the single fp32 rounding.
    t = e4m3.quotient_f32(np.float32(1.0), 3.0)
    assert t.dtype == np.float32 and t == np.float32(1.0) / np.float32(3.0)


def test_decode_scale():
    codes = np.array([0x38, 0x7E, 0x01], dtype=np.uint8)
    out = e4m3.decode(codes, 0.5)
    assert list(out) == [0.5, 224.0, 2.0 ** -10]
