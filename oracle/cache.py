"""Paged cache addressing and the slot writer -- test oracle.

Test infrastructure only (see the package docstring).

Layout.  The pages only say the pages are head-major ("libmir-metal 0.2.0,
src/native/trace/kv.rs", ``fn build``); the byte layout inside a
(block, head) page is fixed by the library's ABI, and the oracle stores
exactly those bytes so that writes can be compared one for one:

* key pool   ``[num_blocks][num_kv_heads][head_dim/8][block_size][8]``:
  row t, dimension d of a page sits at ``((d // 8) * block_size + t) * 8 + d % 8``;
* value pool ``[num_blocks][num_kv_heads][block_size/8][head_dim][8]``: the
  page's rows in groups of 8; row t, dimension d sits at
  ``((t // 8) * head_dim + d) * 8 + t % 8``.  (A block size that is not a
  multiple of 8, which only the oracle's own small tests use, makes one
  group of ``block_size`` rows: ``[1][head_dim][block_size]``.)

The helpers :func:`put_row` / :func:`get_row` are the only places that know
this layout; everything else works with logical rows ``[num_kv_heads, D]``.

Element formats, all held as raw bits so that writes can be compared byte for
byte:

* ``"f16"``  -- IEEE binary16, stored as uint16 bits;
* ``"bf16"`` -- bfloat16 (the top half of an fp32), stored as uint16 bits;
* ``"e4m3"`` -- OCP E4M3 codes, stored as uint8 (see :mod:`oracle.e4m3`);
* ``"int8"`` -- symmetric per-(token, KV head) int8 codes, stored as int8,
  with one fp32 scale per (block, head, row) in separate scale pools
  ``[num_blocks][num_kv_heads][block_size]`` (see :mod:`oracle.int8`).
  For this format the ``k_scale`` / ``v_scale`` arguments below are those
  scale pools instead of per-tensor floats.

The writer is the cache-slot operation the "Optimization plans" discussion
(mistral.rs discussion 46, "Update" post) calls ``reshape_and_cache``: token n
with slot s >= 0 lands in block s // block_size, row s % block_size, for every
KV head; nothing else in the pool changes.  Negative slots are skipped (a
reading: the pages do not say how padding tokens are marked).
"""

from __future__ import annotations

import numpy as np

from . import e4m3
from . import int8


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
    if fmt == "int8":
        return bits.astype(np.int8).astype(np.float64)
    raise ValueError(f"unknown format {fmt!r}")


def storage_dtype(fmt: str):
    return {"e4m3": np.uint8, "int8": np.int8}.get(fmt, np.uint16)


def empty_scale_pools(num_blocks: int, num_kv_heads: int, block_size: int,
                      fill: float = 0.0):
    """Per-row fp32 scale pools of an int8 cache (K and V)."""
    k = np.full((num_blocks, num_kv_heads, block_size), fill, dtype=np.float32)
    return k, k.copy()


def empty_pools(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                fmt: str, fill: int = 0):
    """Key and value pools in their physical layouts, every element = ``fill``."""
    if head_dim % 8:
        raise ValueError("head_dim must be a multiple of 8")
    dt = storage_dtype(fmt)
    tg = value_group(block_size)
    k = np.full((num_blocks, num_kv_heads, head_dim // 8, block_size, 8), fill, dtype=dt)
    v = np.full((num_blocks, num_kv_heads, block_size // tg, head_dim, tg), fill, dtype=dt)
    return k, v


def value_group(block_size: int) -> int:
    """Rows per group of a value page: 8, or the whole block when the
    block size is not a multiple of 8."""
    return 8 if block_size % 8 == 0 else block_size


def pool_geometry(key_cache):
    """(num_blocks, num_kv_heads, block_size, head_dim) of a key pool."""
    nb, hkv, d8, bs, _ = key_cache.shape
    return nb, hkv, bs, d8 * 8


def put_row(key_cache, value_cache, blk: int, off: int, k_row, v_row) -> None:
    """Store one token's K and V rows ``[Hkv, D]`` at (block, row)."""
    hkv, d8 = key_cache.shape[1], key_cache.shape[2]
    tg = value_cache.shape[4]
    key_cache[blk, :, :, off, :] = np.asarray(k_row).reshape(hkv, d8, 8)
    value_cache[blk, :, off // tg, :, off % tg] = np.asarray(v_row)


def get_row(key_cache, value_cache, blk: int, off: int):
    """One token's stored K and V rows ``[Hkv, D]`` at (block, row)."""
    hkv, d8 = key_cache.shape[1], key_cache.shape[2]
    tg = value_cache.shape[4]
    k = key_cache[blk, :, :, off, :].reshape(hkv, d8 * 8)
    v = value_cache[blk, :, off // tg, :, off % tg]
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
                      act_fmt: str, cache_fmt: str, k_scale=1.0, v_scale=1.0) -> None:
    """Write tokens into the pools in place.

    key_bits, value_bits: ``[T, Hkv, D]`` activation bits.
    key_cache, value_cache: pools from :func:`empty_pools`, updated.
    slot_mapping: ``[T]`` ints; ``s >= 0`` writes to block ``s // BS``, row
    ``s % BS``; ``s < 0`` is skipped.
    cache_fmt "int8": k_scale / v_scale are the scale pools, updated with one
    scale per written (row, head).
    """
    bs = pool_geometry(key_cache)[2]
    slots = np.asarray(slot_mapping).reshape(-1)
    for n, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        blk, off = s // bs, s % bs
        if cache_fmt == "int8":
            kc, ksc = int8.quantize_rows(bits_to_f64(key_bits[n], act_fmt).astype(np.float32))
            vc, vsc = int8.quantize_rows(bits_to_f64(value_bits[n], act_fmt).astype(np.float32))
            put_row(key_cache, value_cache, blk, off, kc, vc)
            k_scale[blk, :, off] = ksc
            v_scale[blk, :, off] = vsc
            continue
        put_row(key_cache, value_cache, blk, off,
                encode_tokens(key_bits[n], act_fmt, cache_fmt, k_scale),
                encode_tokens(value_bits[n], act_fmt, cache_fmt, v_scale))


def gather_f64(key_cache, value_cache, block_table_row, length: int, fmt: str,
               k_scale=1.0, v_scale=1.0):
    """Logical rows 0..length-1 of one sequence as fp64 K and V ``[length, Hkv, D]``.

    Walks the block table token by token; for E4M3 the code values are
    multiplied by the per-tensor scales in fp64, for int8 by each row's own
    scale (``k_scale`` / ``v_scale`` are then the scale pools).
    """
    _, hkv, bs, d = pool_geometry(key_cache)
    ks, vs, kss, vss = [], [], [], []
    for t in range(length):
        phys = int(block_table_row[t // bs])
        k, v = get_row(key_cache, value_cache, phys, t % bs)
        ks.append(k)
        vs.append(v)
        if fmt == "int8":
            kss.append(k_scale[phys, :, t % bs])
            vss.append(v_scale[phys, :, t % bs])
    if not ks:
        z = np.zeros((0, hkv, d), dtype=np.float64)
        return z, z.copy()
    if fmt == "int8":
        return int8.decode(np.stack(ks), np.stack(kss)), int8.decode(np.stack(vs), np.stack(vss))
    kv = bits_to_f64(np.stack(ks), fmt)
    vv = bits_to_f64(np.stack(vs), fmt)
    if fmt == "e4m3":
        kv = kv * np.float64(np.float32(k_scale))
        vv = vv * np.float64(np.float32(v_scale))
    return kv, vv


def copy_blocks(key_cache, value_cache, block_mapping, k_scales=None, v_scales=None) -> None:
    """Copy whole blocks (every KV head, K and V, and an int8 cache's row
    scales) from ``src`` to ``dst`` for each pair of ``block_mapping``
    ``[N, 2]``, in place.

    This is the block copy that copy-on-write of a shared, partially filled
    block needs (prefix caching with shared blocks: "PagedAttention in
    mistral.rs", prefix caching notes; "libmir-metal 0.2.0,
    src/native/trace/kv.rs", fn build, copy-on-write page maps).  Sources
    are read before any destination is written.
    """
    pairs = [(int(a), int(b)) for a, b in np.asarray(block_mapping).reshape(-1, 2)]
    src_k = {a: key_cache[a].copy() for a, _ in pairs}
    src_v = {a: value_cache[a].copy() for a, _ in pairs}
    src_ks = {a: k_scales[a].copy() for a, _ in pairs} if k_scales is not None else None
    src_vs = {a: v_scales[a].copy() for a, _ in pairs} if v_scales is not None else None
    for a, b in pairs:
        key_cache[b] = src_k[a]
        value_cache[b] = src_v[a]
        if src_ks is not None:
            k_scales[b] = src_ks[a]
            v_scales[b] = src_vs[a]
