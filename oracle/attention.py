"""Paged decode, rolling-buffer decode, chunked prefill and the split merge.

Test infrastructure only (see the package docstring).  Everything is fp64.

What is computed is the textbook definition of scaled dot-product attention,
``softmax(scale * q k^T) v``, with the keys and values fetched through a block
table ("PagedAttention in mistral.rs": the cache is cut into fixed-size token
blocks and each sequence reaches its blocks through a table).  The paged
method is exact up to rounding order, so the oracle is the definition.

Readings where the pages are silent (each listed in the design notes):

* Query head h reads KV head ``h // (Hq // Hkv)`` (contiguous groups).
* ``context_lens[b]`` counts the token being decoded: the writer stores it
  first, then attention reads it (write-then-attend, as the "Update" post of
  mistral.rs discussion 46 orders the two operations).
* An empty context gives an all-zero output.
* Rolling buffer ("Rolling buffer cache", llama.cpp discussion 3581, opening
  post): position i sits at ring slot i mod W; a W-slot ring written before
  attending holds positions i-W+1 .. i, so the query attends to W keys.  The
  ring is read in slot order; softmax does not depend on key order.
* Chunked prefill: query j of a chunk of C tokens appended to a context of
  total length ctx sits at absolute position ctx - C + j and sees keys
  0 .. ctx - C + j (causal).
"""

from __future__ import annotations

import numpy as np

from .cache import bits_to_f64, gather_f64, get_row, pool_geometry, slot_of


def softmax_attend(q, k, v, scale: float):
    """softmax(scale * k q) weighted sum of v, for one query vector.

    q: ``[D]``; k, v: ``[L, D]``; returns ``[D]`` (zeros when L == 0).
    """
    if k.shape[0] == 0:
        return np.zeros(v.shape[1], dtype=np.float64)
    s = scale * (k @ q)
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ v) / np.sum(p)


def decode(query_bits, act_fmt: str, key_cache, value_cache, cache_fmt: str,
           block_tables, context_lens, scale: float, k_scale: float = 1.0,
           v_scale: float = 1.0, window: int = 0):
    """Paged decode: one query token per sequence.

    query_bits: ``[B, Hq, D]`` activation bits.  Pools as in :mod:`oracle.cache`.
    block_tables: ``[B, MBPS]``; context_lens: ``[B]``.
    window == 0: attend to logical rows 0..L-1 with L = context_lens[b].
    window  > 0: the table addresses a ring of ``window`` rows; attend to ring
    rows 0..min(L, window)-1.
    k_scale / v_scale: per-tensor scales of an E4M3 cache, or the per-row
    scale pools of an int8 cache (see :mod:`oracle.cache`).
    Returns fp64 ``[B, Hq, D]``.
    """
    q = bits_to_f64(query_bits, act_fmt)
    B, Hq, D = q.shape
    Hkv = key_cache.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if window > 0:
            L = min(L, window)
        k, v = gather_f64(key_cache, value_cache, block_tables[b], L, cache_fmt, k_scale,
                          v_scale)
        for h in range(Hq):
            g = h // group
            out[b, h] = softmax_attend(q[b, h], k[:, g, :], v[:, g, :], scale)
    return out


def prefill_chunk(query_bits, act_fmt: str, cu_q_lens, key_cache, value_cache,
                  cache_fmt: str, block_tables, context_lens, scale: float,
                  k_scale: float = 1.0, v_scale: float = 1.0):
    """Chunked prefill with a causal mask over prefix + chunk.

    query_bits: ``[total_q, Hq, D]`` packed; sequence b owns rows
    ``cu_q_lens[b] .. cu_q_lens[b+1]-1``.  context_lens[b] includes the chunk.
    Returns fp64 ``[total_q, Hq, D]``.
    """
    q = bits_to_f64(query_bits, act_fmt)
    total, Hq, D = q.shape
    Hkv = key_cache.shape[1]
    group = Hq // Hkv
    out = np.zeros((total, Hq, D), dtype=np.float64)
    B = len(cu_q_lens) - 1
    for b in range(B):
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        C = q1 - q0
        ctx = int(context_lens[b])
        k, v = gather_f64(key_cache, value_cache, block_tables[b], ctx, cache_fmt, k_scale,
                          v_scale)
        for j in range(C):
            i = ctx - C + j  # absolute position of this query
            for h in range(Hq):
                g = h // group
                out[q0 + j, h] = softmax_attend(q[q0 + j, h], k[: i + 1, g, :],
                                                v[: i + 1, g, :], scale)
    return out


def prefill_chunk_window(query_bits, act_fmt: str, key_bits, value_bits, cu_q_lens,
                         key_cache, value_cache, cache_fmt: str, block_tables, context_lens,
                         scale: float, window: int, rows=None, k_scale=1.0, v_scale=1.0):
    """Chunked prefill of a sliding-window layer whose cache is a ring of
    ``window`` rows ("Rolling buffer cache", opening post: position i lives
    in ring row i mod W).

    Reading (the pages only say the ring exists and that a token attends to
    the last W positions): the chunk has not been written into the ring
    yet, because its later tokens would overwrite ring rows that its earlier
    queries still need.  Query j of sequence b sits at position
    ``i = ctx - C + j`` and attends to positions ``max(0, i - W + 1) .. i``:
    those before the chunk (``< ctx - C``) from the ring, the chunk's own
    from ``key_bits`` / ``value_bits`` (``[total_q, Hkv, D]``, packed like
    the queries).

    A quantised ring is read as the cache stores it: E4M3 codes times the
    per-tensor scales (``k_scale``, ``v_scale``; "PagedAttention in
    mistral.rs", section "KV Cache Quantization"), INT8 codes times their
    row's own scale (``k_scale`` / ``v_scale`` are then the scale pools;
    "libmir-metal 0.2.0, src/native/trace/kv.rs", fn build).  The chunk's own
    K/V are the activations as given, not yet quantised (the same reading as
    above: they are not in the cache yet).

    ``rows``: optionally, the (b, j) pairs to compute (the others stay 0),
    for spot checks of workloads too large to compute whole.
    """
    q = bits_to_f64(query_bits, act_fmt)
    kn = bits_to_f64(key_bits, act_fmt)
    vn = bits_to_f64(value_bits, act_fmt)
    total, Hq, D = q.shape
    group = Hq // key_cache.shape[1]
    bs = pool_geometry(key_cache)[2]
    out = np.zeros((total, Hq, D), dtype=np.float64)
    for b in range(len(cu_q_lens) - 1):
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        C = q1 - q0
        ctx = int(context_lens[b])
        start = ctx - C                      # first position of the chunk
        for j in range(C):
            if rows is not None and (b, j) not in rows:
                continue
            i = start + j
            ks, vs = [], []
            for pos in range(max(0, i - window + 1), i + 1):
                if pos < start:
                    slot = slot_of(block_tables[b], pos % window, bs)
                    k_row, v_row = get_row(key_cache, value_cache, slot // bs, slot % bs)
                    k_row, v_row = bits_to_f64(k_row, cache_fmt), bits_to_f64(v_row, cache_fmt)
                    if cache_fmt == "e4m3":
                        k_row = k_row * np.float64(np.float32(k_scale))
                        v_row = v_row * np.float64(np.float32(v_scale))
                    elif cache_fmt == "int8":
                        k_row = k_row * np.asarray(k_scale[slot // bs, :, slot % bs],
                                                   np.float64)[:, None]
                        v_row = v_row * np.asarray(v_scale[slot // bs, :, slot % bs],
                                                   np.float64)[:, None]
                    ks.append(k_row)
                    vs.append(v_row)
                else:
                    ks.append(kn[q0 + pos - start])
                    vs.append(vn[q0 + pos - start])
            k = np.stack(ks)
            v = np.stack(vs)
            for h in range(Hq):
                out[q0 + j, h] = softmax_attend(q[q0 + j, h], k[:, h // group, :],
                                                v[:, h // group, :], scale)
    return out


def partial(q, k, v, scale: float):
    """Unnormalised partial result of one key partition.

    Returns (m, l, o): m = max score, l = sum of exp(s - m),
    o = sum of exp(s - m) * v.  An empty partition gives (-inf, 0, 0).
    """
    if k.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(v.shape[1], dtype=np.float64)
    s = scale * (k @ q)
    m = np.max(s)
    p = np.exp(s - m)
    return m, np.sum(p), p @ v


def merge(parts):
    """Combine partition partials (m_p, l_p, o_p) into the attention output.

    M = max m_p; w_p = exp(m_p - M); out = sum w_p o_p / sum w_p l_p.
    """
    live = [(m, l, o) for (m, l, o) in parts if np.isfinite(m)]
    if not live:
        return np.zeros_like(parts[0][2])
    M = max(m for m, _, _ in live)
    num = sum(np.exp(m - M) * o for m, _, o in live)
    den = sum(np.exp(m - M) * l for m, l, _ in live)
    return num / den
