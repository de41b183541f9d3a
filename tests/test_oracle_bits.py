"""Pin of ``oracle.cache.bits_to_f64``, the function every oracle input goes
through: every 16-bit pattern of bf16 and f16, and every INT8 and E4M3 code,
against torch's own reinterpretation and widening (``Tensor.view(dtype)``
then ``.to(float64)``), an implementation that shares nothing with the
oracle's bit arithmetic.  NaN patterns must give NaN; every other pattern the
same value, signed zeros and infinities included.
"""

import numpy as np
import pytest
import torch

from oracle import cache


def _same(a: np.ndarray, b: np.ndarray) -> None:
    nan_a, nan_b = np.isnan(a), np.isnan(b)
    assert np.array_equal(nan_a, nan_b), "NaN patterns differ"
    ok = ~nan_a
    assert np.array_equal(a[ok], b[ok])
    # Signed zeros and infinities keep their signs.
    assert np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
@pytest.mark.parametrize("fmt,dtype", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_every_16bit_pattern(fmt, dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = cache.bits_to_f64(bits, fmt)
    ref = torch.from_numpy(bits.view(np.int16)).view(dtype).to(torch.float64).numpy()
    assert ours.dtype == np.float64 and ours.shape == bits.shape
    _same(ours, ref)
    # The count of NaN patterns is fixed by the formats: exponent all ones,
    # mantissa non-zero, either sign.
    man = 7 if fmt == "bf16" else 10
    assert int(np.isnan(ours).sum()) == 2 * ((1 << man) - 1)


def test_every_int8_code():
    codes = np.arange(-128, 128, dtype=np.int8)
    ours = cache.bits_to_f64(codes, "int8")
    ref = torch.from_numpy(codes).to(torch.float64).numpy()
    _same(ours, ref)


def test_every_e4m3_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = cache.bits_to_f64(codes, "e4m3")
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(ours, ref)
    assert int(np.isnan(ours).sum()) == 2          # 0x7f and 0xff only


def test_shape_and_unknown_format():
    bits = np.arange(24, dtype=np.uint16).reshape(2, 3, 4)
    assert cache.bits_to_f64(bits, "bf16").shape == (2, 3, 4)
    with pytest.raises(ValueError):
        cache.bits_to_f64(bits, "fp32")
