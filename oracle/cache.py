"""Paged cache addressing and the slot writer -- test oracle.

Test infrastructure only (see the package docstring).

Layout (a reading of the head-major pages named in "libmir-metal 0.2.0,
src/native/trace/kv.rs", ``fn build``): each cache pool is
``[num_blocks, num_kv_heads, block_size, head_dim]``, so one (block, head)
page is a contiguous run of ``block_size * head_dim`` elements.

Element formats, all held as raw bits so that writes can be compared byte for
byte:

* ``"f16"``  -- IEEE binary16, stored as uint16 bits;
* ``"bf16"`` -- bfloat16 (the top half of an fp32), stored as uint16 bits;
* ``"e4m3"`` -- OCP E4M3 codes, stored as uint8 (see :mod:`oracle.e4m3`).

The writer is the cache-slot operation the "Optimization plans" discussion
(mistral.rs discussion 46, "Update" post) calls ``reshape_and_cache``: token n
with slot s >= 0 lands in block s // block_size, row s % block_size, for every
KV head; nothing else in the pool changes.  Negative slots are skipped (a
reading: the pages do not say how padding tokens are marked).
"""

from __future__ import annotations

import numpy as np

from . import e4m3


def bits_to_f64(bits, fmt: str) -> np.ndarray:
    """fp64 values of an array of stored elements in format ``fmt``."""
    bits = np.asarray(bits)
    if fmt == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    if fmt == "bf16":
        wide = bits.astype(np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if fmt == "e4m3":
        return e4m3.decode(bits, 1.0)
    raise ValueError(f"unknown format {fmt!r}")


def storage_dtype(fmt: str):
    return np.uint8 if fmt == "e4m3" else np.uint16


def slot_of(block_table_row, logical_index: int, block_size: int) -> int:
    """Flat slot holding logical cache index ``logical_index`` of a sequence.

    The table row maps logical block j to a physical block; the slot is
    ``physical * block_size + offset``.
    """
    phys = int(block_table_row[logical_index // block_size])
    return phys * block_size + logical_index % block_size


def encode_tokens(x_bits, act_fmt: str, cache_fmt: str, scale: float):
    """What the writer stores for a batch of activation elements."""
    x_bits = np.asarray(x_bits)
    if cache_fmt == act_fmt:
        return x_bits.astype(storage_dtype(cache_fmt))
    if cache_fmt == "e4m3":
        x32 = bits_to_f64(x_bits, act_fmt).astype(np.float32)  # exact
        return e4m3.encode(x32, scale)
    raise ValueError(f"unsupported cache format {cache_fmt!r} for act {act_fmt!r}")


def reshape_and_cache(key_bits, value_bits, key_cache, value_cache, slot_mapping,
                      act_fmt: str, cache_fmt: str, k_scale: float = 1.0,
                      v_scale: float = 1.0) -> None:
    """Write tokens into the pools in place.

    key_bits, value_bits: ``[T, Hkv, D]`` activation bits.
    key_cache, value_cache: ``[NB, Hkv, BS, D]`` storage arrays, updated.
    slot_mapping: ``[T]`` ints; ``s >= 0`` writes to block ``s // BS``, row
    ``s % BS``; ``s < 0`` is skipped.
    """
    bs = key_cache.shape[2]
    slots = np.asarray(slot_mapping).reshape(-1)
    for n, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = s // bs, s % bs
        key_cache[blk, :, off, :] = encode_tokens(key_bits[n], act_fmt, cache_fmt, k_scale)
        value_cache[blk, :, off, :] = encode_tokens(value_bits[n], act_fmt, cache_fmt, v_scale)


def gather_f64(cache, block_table_row, length: int, fmt: str, scale: float = 1.0):
    """Logical rows 0..length-1 of one sequence as fp64 ``[length, Hkv, D]``.

    Walks the block table token by token; for E4M3 the code values are
    multiplied by the scale in fp64.
    """
    bs = cache.shape[2]
    rows = []
    for t in range(length):
        phys = int(block_table_row[t // bs])
        rows.append(cache[phys, :, t % bs, :])
    if not rows:
        return np.zeros((0, cache.shape[1], cache.shape[3]), dtype=np.float64)
    vals = bits_to_f64(np.stack(rows), fmt)
    if fmt == "e4m3":
        vals = vals * np.float64(np.float32(scale))
    return vals
