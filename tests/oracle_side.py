"""The oracle side of the parity tests: seeded workloads written into the
oracle's own pools with the oracle's writer and attended with the oracle's
attention (``oracle/``), plus a process pool that runs those same functions
over groups of sequences at the benchmark workloads' full sizes.

No torch here: the pool's workers import only numpy, ``oracle`` and this
module.  The pool's workers are forked from a forkserver started (``start``)
before the test process touches the GPU, so no worker inherits GPU state.

Splitting a batch into groups changes nothing the oracle computes: every
group runs the unchanged oracle functions on its own sequences, with the
blocks those sequences own renumbered into a compact pool (a renaming of
block ids, which the paged definition does not depend on), and the groups'
pool blocks are put back at their ids afterwards.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import types

import numpy as np

from oracle import attention as o_attn
from oracle import cache as o_cache
from oracle import pool as o_pool

NAN16 = {"bf16": 0x7FC0, "f16": 0x7E00}
NAN_E4M3 = 0x7F
NAN_F32 = float("nan")


# --------------------------------------------------------------------------- one process


def oracle_pools(wl):
    fill = NAN_E4M3 if wl.cache == "e4m3" else NAN16[wl.cache]
    return o_cache.empty_pools(wl.pool_blocks, wl.Hkv, wl.BS, wl.D, wl.cache, fill)


def _oracle_row(wl, pos):
    return o_pool.ring_index(int(pos), wl.window) if wl.window else int(pos)


def oracle_decode_setup(wl, seqs=None):
    kc, vc = oracle_pools(wl)
    seqs = range(wl.B) if seqs is None else seqs
    for b in seqs:
        n = wl.cached_k[b].shape[0]
        slots = [o_cache.slot_of(wl.block_tables[b], _oracle_row(wl, wl.cached_pos0[b] + t), wl.BS)
                 for t in range(n)]
        o_cache.reshape_and_cache(wl.cached_k[b], wl.cached_v[b], kc, vc, np.array(slots, np.int64),
                                  wl.act, wl.cache, wl.k_scale, wl.v_scale)
    for b in seqs:
        s = o_cache.slot_of(wl.block_tables[b], _oracle_row(wl, wl.new_pos[b]), wl.BS)
        o_cache.reshape_and_cache(wl.new_k[b:b + 1], wl.new_v[b:b + 1], kc, vc, np.array([s]),
                                  wl.act, wl.cache, wl.k_scale, wl.v_scale)
    return kc, vc


def oracle_decode(wl, kc, vc, seqs=None):
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    return o_attn.decode(wl.query[seqs], wl.act, kc, vc, wl.cache, wl.block_tables[seqs],
                         wl.context_lens[seqs], wl.scale, wl.k_scale, wl.v_scale, wl.window)


def oracle_prefill_setup(wl):
    kc, vc = oracle_pools(wl)
    slots = [o_cache.slot_of(wl.block_tables[0], t, wl.BS) for t in range(wl.prefix_len)]
    o_cache.reshape_and_cache(wl.prefix_k, wl.prefix_v, kc, vc, np.array(slots, np.int64),
                              wl.act, wl.cache, wl.k_scale, wl.v_scale)
    for b in range(wl.B):
        C = int(wl.chunk_lens[b])
        slots = [o_cache.slot_of(wl.block_tables[b], wl.prefix_len + t, wl.BS) for t in range(C)]
        o_cache.reshape_and_cache(wl.chunk_k[b], wl.chunk_v[b], kc, vc, np.array(slots, np.int64),
                                  wl.act, wl.cache, wl.k_scale, wl.v_scale)
    return kc, vc


def oracle_prefill(wl, kc, vc):
    return o_attn.prefill_chunk(wl.query, wl.act, wl.cu_q_lens, kc, vc, wl.cache,
                                wl.block_tables, wl.context_lens, wl.scale, wl.k_scale,
                                wl.v_scale)


# INT8 cache: pools of int8 codes plus fp32 scale pools [NB+1, Hkv, BS]; the
# scales start NaN-filled, so a stale row that reaches an output shows up as NaN.

def oracle_pools_i8(wl):
    kc, vc = o_cache.empty_pools(wl.pool_blocks, wl.Hkv, wl.BS, wl.D, "int8", 0x7F)
    ks, vs = o_cache.empty_scale_pools(wl.pool_blocks, wl.Hkv, wl.BS, NAN_F32)
    return kc, vc, ks, vs


def oracle_decode_setup_i8(wl, seqs=None):
    kc, vc, ks, vs = oracle_pools_i8(wl)
    seqs = range(wl.B) if seqs is None else seqs
    for b in seqs:
        n = wl.cached_k[b].shape[0]
        slots = [o_cache.slot_of(wl.block_tables[b], _oracle_row(wl, wl.cached_pos0[b] + t), wl.BS)
                 for t in range(n)]
        o_cache.reshape_and_cache(wl.cached_k[b], wl.cached_v[b], kc, vc, np.array(slots, np.int64),
                                  wl.act, "int8", ks, vs)
    for b in seqs:
        s = o_cache.slot_of(wl.block_tables[b], _oracle_row(wl, wl.new_pos[b]), wl.BS)
        o_cache.reshape_and_cache(wl.new_k[b:b + 1], wl.new_v[b:b + 1], kc, vc, np.array([s]),
                                  wl.act, "int8", ks, vs)
    return kc, vc, ks, vs


def oracle_decode_i8(wl, pools, seqs=None):
    kc, vc, ks, vs = pools
    seqs = list(range(wl.B)) if seqs is None else list(seqs)
    return o_attn.decode(wl.query[seqs], wl.act, kc, vc, "int8", wl.block_tables[seqs],
                         wl.context_lens[seqs], wl.scale, ks, vs, wl.window)


def oracle_prefill_setup_i8(wl):
    kc, vc, ks, vs = oracle_pools_i8(wl)
    slots = [o_cache.slot_of(wl.block_tables[0], t, wl.BS) for t in range(wl.prefix_len)]
    o_cache.reshape_and_cache(wl.prefix_k, wl.prefix_v, kc, vc, np.array(slots, np.int64),
                              wl.act, "int8", ks, vs)
    for b in range(wl.B):
        C = int(wl.chunk_lens[b])
        slots = [o_cache.slot_of(wl.block_tables[b], wl.prefix_len + t, wl.BS) for t in range(C)]
        o_cache.reshape_and_cache(wl.chunk_k[b], wl.chunk_v[b], kc, vc, np.array(slots, np.int64),
                                  wl.act, "int8", ks, vs)
    return kc, vc, ks, vs


def oracle_prefill_i8(wl, pools):
    kc, vc, ks, vs = pools
    return o_attn.prefill_chunk(wl.query, wl.act, wl.cu_q_lens, kc, vc, "int8",
                                wl.block_tables, wl.context_lens, wl.scale, ks, vs)


def window_ring_setup(wl, seqs=None):
    """The rings of a window-prefill workload, written position by position
    with the oracle's writer (ring row = position mod W).  Returns the pools
    and the scales the attention reads (per-tensor, or the INT8 scale pools)."""
    seqs = range(wl.B) if seqs is None else seqs
    if wl.cache == "int8":
        kc, vc, ks, vs = oracle_pools_i8(wl)
    else:
        fill = NAN_E4M3 if wl.cache == "e4m3" else NAN16[wl.act]
        kc, vc = o_cache.empty_pools(wl.pool_blocks, wl.Hkv, wl.BS, wl.D, wl.cache, fill)
        ks, vs = wl.k_scale, wl.v_scale
    for b in seqs:
        pos = range(int(wl.hist_pos0[b]), int(wl.hist_lens[b]))
        slots = [o_cache.slot_of(wl.block_tables[b], o_pool.ring_index(p, wl.window), wl.BS)
                 for p in pos]
        o_cache.reshape_and_cache(wl.hist_k[b], wl.hist_v[b], kc, vc, np.array(slots, np.int64),
                                  wl.act, wl.cache, ks, vs)
    return kc, vc, ks, vs


# --------------------------------------------------------------------------- process pool

_CTX = None


def workers() -> int:
    """Worker processes: the CPUs this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def start() -> None:
    """Start the forkserver the pool's workers are forked from.  Call before
    the GPU is initialised (the test session does, at collection)."""
    global _CTX
    if _CTX is not None:
        return
    _CTX = mp.get_context("forkserver")
    _CTX.set_forkserver_preload(["numpy", "oracle.attention", "oracle.cache", "oracle_side"])
    from multiprocessing import forkserver
    forkserver.ensure_running()


def pmap(fn, jobs):
    start()
    n = min(workers(), len(jobs))
    if n <= 1:
        return [fn(j) for j in jobs]
    with _CTX.Pool(n) as p:
        return p.map(fn, jobs, chunksize=1)


def _groups(weights, n):
    """Indices split into at most n groups of about equal total weight."""
    order = np.argsort(-np.asarray(weights, dtype=np.float64), kind="stable")
    groups = [[] for _ in range(n)]
    load = np.zeros(n)
    for i in order:
        g = int(np.argmin(load))
        groups[g].append(int(i))
        load[g] += float(weights[i])
    return [sorted(g) for g in groups if g]


def _compact(tables, nblk, pool_blocks):
    """Renumber the first nblk[r] entries of each table row into 0..n-1.
    Returns (new tables, the original ids of the compact blocks)."""
    used = np.unique(np.concatenate([tables[r, :nblk[r]] for r in range(len(nblk))]))
    assert used.size == 0 or (used.min() >= 0 and used.max() < pool_blocks)
    local = np.full(pool_blocks, -1, dtype=np.int64)
    local[used] = np.arange(used.size)
    out = np.zeros_like(tables)
    for r in range(len(nblk)):
        out[r, :nblk[r]] = local[tables[r, :nblk[r]]]
    return out, used


def _decode_job(job):
    wl = types.SimpleNamespace(**job)
    if wl.cache == "int8":
        pools = oracle_decode_setup_i8(wl)
        out = oracle_decode_i8(wl, pools)
    else:
        pools = oracle_decode_setup(wl)
        out = oracle_decode(wl, *pools)
    return pools, out


def full_decode(wl):
    """The oracle's pools (every block the batch writes) and outputs (every
    sequence) of a decode workload, the work spread over sequence groups.
    Blocks are owned by one sequence each (asserted)."""
    L = wl.context_lens.astype(np.int64)
    if wl.window:
        L = np.minimum(L, wl.window)
    nblk = -(-L // wl.BS)
    jobs, ids = [], []
    groups = _groups(L + 64, 4 * workers())
    for g in groups:
        tables, used = _compact(wl.block_tables[g], nblk[g], wl.pool_blocks)
        ids.append(used)
        jobs.append(dict(
            act=wl.act, cache=wl.cache, B=len(g), Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, BS=wl.BS,
            window=wl.window, scale=wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
            pool_blocks=int(used.size), block_tables=tables, context_lens=wl.context_lens[g],
            query=wl.query[g], cached_pos0=wl.cached_pos0[g],
            cached_k=[wl.cached_k[b] for b in g], cached_v=[wl.cached_v[b] for b in g],
            new_pos=wl.new_pos[g], new_k=wl.new_k[g], new_v=wl.new_v[g]))
    allids = np.concatenate(ids)
    assert np.unique(allids).size == allids.size, "a block is shared between sequences"
    res = pmap(_decode_job, jobs)
    pools = oracle_pools_i8(wl) if wl.cache == "int8" else oracle_pools(wl)
    out = np.zeros((wl.B, wl.Hq, wl.D), dtype=np.float64)
    for g, used, (gp, gout) in zip(groups, ids, res):
        for full, part in zip(pools, gp):
            full[used] = part
        out[g] = gout
    return pools, out


def _prefill_job(job):
    wl = types.SimpleNamespace(**job)
    if wl.cache == "int8":
        pools = oracle_prefill_setup_i8(wl)
        out = oracle_prefill_i8(wl, pools)
    else:
        pools = oracle_prefill_setup(wl)
        out = oracle_prefill(wl, *pools)
    return pools, out


def full_prefill(wl):
    """The oracle's pools and every output row of a shared-prefix prefill
    workload, one job per sequence (each job writes the shared prefix into
    its own compact pool through its own table row, which holds the same
    shared blocks as row 0; the copies are checked equal when put back)."""
    nsh = wl.prefix_len // wl.BS
    assert all(np.array_equal(wl.block_tables[b, :nsh], wl.block_tables[0, :nsh])
               for b in range(wl.B))
    jobs, ids = [], []
    for b in range(wl.B):
        C = int(wl.chunk_lens[b])
        ctx = int(wl.context_lens[b])
        tables, used = _compact(wl.block_tables[b:b + 1], [-(-ctx // wl.BS)], wl.pool_blocks)
        ids.append(used)
        q0, q1 = int(wl.cu_q_lens[b]), int(wl.cu_q_lens[b + 1])
        jobs.append(dict(
            act=wl.act, cache=wl.cache, B=1, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, BS=wl.BS,
            scale=wl.scale, k_scale=wl.k_scale, v_scale=wl.v_scale, pool_blocks=int(used.size),
            prefix_len=wl.prefix_len, prefix_k=wl.prefix_k, prefix_v=wl.prefix_v,
            chunk_lens=wl.chunk_lens[b:b + 1], chunk_k=[wl.chunk_k[b]], chunk_v=[wl.chunk_v[b]],
            cu_q_lens=np.array([0, C], np.int32), context_lens=wl.context_lens[b:b + 1],
            block_tables=tables, query=wl.query[q0:q1]))
    res = pmap(_prefill_job, jobs)
    pools = oracle_pools_i8(wl) if wl.cache == "int8" else oracle_pools(wl)
    seen = np.zeros(wl.pool_blocks, dtype=bool)
    out = np.zeros((wl.total_q, wl.Hq, wl.D), dtype=np.float64)
    for b, (used, (gp, gout)) in enumerate(zip(ids, res)):
        for full, part in zip(pools, gp):
            again = seen[used]
            if again.any():
                a, p = full[used[again]], part[again]
                assert np.array_equal(a.view(np.uint8), p.view(np.uint8)), "shared blocks differ"
            full[used] = part
        seen[used] = True
        out[int(wl.cu_q_lens[b]):int(wl.cu_q_lens[b + 1])] = gout
    return pools, out


def _window_job(job):
    rows = job.pop("rows")
    wl = types.SimpleNamespace(**job)
    kc, vc, ks, vs = window_ring_setup(wl)
    ref = o_attn.prefill_chunk_window(wl.query, wl.act, wl.chunk_k, wl.chunk_v, wl.cu_q_lens,
                                      kc, vc, wl.cache, wl.block_tables, wl.context_lens,
                                      wl.scale, wl.window, rows={(0, j) for j in rows},
                                      k_scale=ks, v_scale=vs)
    return (kc, vc, ks, vs), ref[rows]


def window_prefill_rows(wl, rows_of, parts: int = 4):
    """The oracle's rings (every sequence) and its outputs at query rows
    ``rows_of[b]`` (chunk-relative) of every sequence and head, a job per
    sequence and part of its rows.  Returns (pools, {(b, j): out[Hq, D]})."""
    jobs, meta = [], []
    for b in range(wl.B):
        nb = wl.block_tables.shape[1]
        tables, used = _compact(wl.block_tables[b:b + 1], [nb], wl.pool_blocks)
        q0, q1 = int(wl.cu_q_lens[b]), int(wl.cu_q_lens[b + 1])
        sel = sorted(rows_of[b])
        for part in np.array_split(np.asarray(sel, dtype=np.int64), parts):
            if part.size == 0:
                continue
            job = dict(act=wl.act, cache=wl.cache, B=1, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                       BS=wl.BS, window=wl.window, scale=wl.scale, pool_blocks=int(used.size),
                       hist_lens=wl.hist_lens[b:b + 1], hist_pos0=wl.hist_pos0[b:b + 1],
                       chunk_lens=wl.chunk_lens[b:b + 1], cu_q_lens=np.array([0, q1 - q0]),
                       context_lens=wl.context_lens[b:b + 1], block_tables=tables,
                       query=wl.query[q0:q1], chunk_k=wl.chunk_k[q0:q1],
                       chunk_v=wl.chunk_v[q0:q1], hist_k=[wl.hist_k[b]], hist_v=[wl.hist_v[b]],
                       k_scale=wl.k_scale, v_scale=wl.v_scale, rows=[int(x) for x in part])
            jobs.append(job)
            meta.append((b, used, [int(x) for x in part]))
    res = pmap(_window_job, jobs)
    if wl.cache == "int8":
        pools = list(oracle_pools_i8(wl))
    else:
        fill = NAN_E4M3 if wl.cache == "e4m3" else NAN16[wl.act]
        pools = list(o_cache.empty_pools(wl.pool_blocks, wl.Hkv, wl.BS, wl.D, wl.cache, fill))
    out = {}
    for (b, used, part), (gp, ref) in zip(meta, res):
        for i, (full, p) in enumerate(zip(pools, gp[:len(pools)])):
            full[used] = p
        for j, r in zip(part, ref):
            out[(b, j)] = r
    return tuple(pools), out
