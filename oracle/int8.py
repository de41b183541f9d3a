"""INT8 per-token/head cache codec -- test oracle.

Test infrastructure only (see the package docstring).

"libmir-metal 0.2.0, src/native/trace/kv.rs", ``fn build``: a quantised KV
cache keeps full-attention K and V as packed INT8 pages with one FP32 scale
per token and head, and the paged attention kernels dequantise inside the
attention (for prefill and for decode).  The page gives no arithmetic; this
module takes the plainest reading of "per-token/head INT8 with an FP32
scale", symmetric quantisation of each (token, KV head) row of D values:

* ``scale = fp32(max_d |x_d|) / fp32(127)`` (IEEE single division);
* ``code_d = clamp(round_half_even(fp32(x_d) / scale), -127, 127)`` with IEEE
  single division; a row of zeros has scale 0 and all codes 0;
* the value a code stands for is ``code * scale``.

K and V rows are quantised separately, each with its own scale.
"""

from __future__ import annotations

import numpy as np

QMAX = 127


def row_scale(x_f32) -> np.float32:
    """The FP32 scale of one row of fp32 values."""
    x = np.asarray(x_f32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    return np.float32(amax / np.float32(QMAX))


def encode_row(x_f32, scale) -> np.ndarray:
    """int8 codes of one row at a given scale (round half to even, clamped)."""
    x = np.asarray(x_f32, dtype=np.float32)
    scale = np.float32(scale)
    if scale == 0:
        return np.zeros(x.shape, dtype=np.int8)
    t = (x / scale).astype(np.float32)          # IEEE single division
    q = np.rint(t)                              # ties to even
    return np.clip(q, -QMAX, QMAX).astype(np.int8)


def quantize_rows(x_f32):
    """Codes ``[..., D]`` int8 and scales ``[...]`` fp32 of every row."""
    x = np.asarray(x_f32, dtype=np.float32)
    lead = x.shape[:-1]
    flat = x.reshape(-1, x.shape[-1])
    codes = np.empty(flat.shape, dtype=np.int8)
    scales = np.empty(flat.shape[0], dtype=np.float32)
    for i, row in enumerate(flat):
        scales[i] = row_scale(row)
        codes[i] = encode_row(row, scales[i])
    return codes.reshape(x.shape), scales.reshape(lead)


def decode(codes, scales) -> np.ndarray:
    """fp64 values ``code * scale``; scales broadcast over the last axis."""
    return (np.asarray(codes, dtype=np.float64)
            * np.asarray(scales, dtype=np.float64)[..., None])
