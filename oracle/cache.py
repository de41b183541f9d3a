"""Paged cache addressing and the slot writer -- test oracle.

Test infrastructure only (see the package docstring).

Layout.  The pages only say the pages are head-major ("libmir-metal 0.2.0,
src/native/trace/kv.rs", ``fn build``); the byte layout inside a
(block, head) page is fixed by the library's ABI, and the oracle stores
exactly those bytes so that writes can be compared one for one:

* key pool   ``[num_blocks][num_kv_heads][head_dim/8][block_size][8]``:
  row t, dimension d of a page sits at ``((d // 8) * block_size + t) * 8 + d % 8``;
* value pool ``[num_blocks][num_kv_heads][head_dim][block_size]``: row t,
  dimension d sits at ``d * block_size + t`` (the page is stored transposed).

The helpers :func:`put_row` / :func:`get_row` are the only places that know
this layout; everything else works with logical rows ``[num_kv_heads, D]``.

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


def empty_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                fmt: str, fill: int = 0):
    """Key and value pools in their physical layouts, every element = ``fill``."""
    if head_dim % 8:
        raise ValueError("head_dim must be a multiple of 8")
    dt = storage_dtype(fmt)
    k = np.full((num_blocks, num_kv_heads, head_dim // 8, block_size, 8), fill, dtype=dt)
    v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill, dtype=dt)
    return k, v


def pool_geometry(key_cache):
    """(num_blocks, num_kv_heads, block_size, head_dim) of a key pool."""
    nb, hkv, d8, bs, _ = key_cache.shape
    return nb, hkv, bs, d8 * 8


def put_row(key_cache, value_cache, blk: int, off: int, k_row, v_row) -> None:
    """Store one token's K and V rows ``[Hkv, D]`` at (block, row)."""
    hkv, d8 = key_cache.shape[1], key_cache.shape[2]
    key_cache[blk, :, :, off, :] = np.asarray(k_row).reshape(hkv, d8, 8)
    value_cache[blk, :, :, off] = np.asarray(v_row)


def get_row(key_cache, value_cache, blk: int, off: int):
    """One token's stored K and V rows ``[Hkv, D]`` at (block, row)."""
    hkv, d8 = key_cache.shape[1], key_cache.shape[2]
    k = key_cache[blk, :, :, off, :].reshape(hkv, d8 * 8)
    v = value_cache[blk, :, :, off]
    return k, v


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
    key_cache, value_cache: pools from :func:`empty_pools`, updated.
    slot_mapping: ``[T]`` ints; ``s >= 0`` writes to block ``s // BS``, row
    ``s % BS``; ``s < 0`` is skipped.
    """
    bs = pool_geometry(key_cache)[2]
    slots = np.asarray(slot_mapping).reshape(-1)
    for n, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        put_row(key_cache, value_cache, s // bs, s % bs,
                encode_tokens(key_bits[n], act_fmt, cache_fmt, k_scale),
                encode_tokens(value_bits[n], act_fmt, cache_fmt, v_scale))


def gather_f64(key_cache, value_cache, block_table_row, length: int, fmt: str,
               k_scale: float = 1.0, v_scale: float = 1.0):
    """Logical rows 0..length-1 of one sequence as fp64 K and V ``[length, Hkv, D]``.

    Walks the block table token by token; for E4M3 the code values are
    multiplied by the scales in fp64.
    """
    _, hkv, bs, d = pool_geometry(key_cache)
    ks, vs = [], []
    for t in range(length):
        phys = int(block_table_row[t // bs])
        k, v = get_row(key_cache, value_cache, phys, t % bs)
        ks.append(k)
        vs.append(v)
    if not ks:
        z = np.zeros((0, hkv, d), dtype=np.float64)
        return z, z.copy()
    kv = bits_to_f64(np.stack(ks), fmt)
    vv = bits_to_f64(np.stack(vs), fmt)
    if fmt == "e4m3":
        kv = kv * np.float64(np.float32(k_scale))
        vv = vv * np.float64(np.float32(v_scale))
    return kv, vv
