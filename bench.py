#!/usr/bin/env python3
"""Paged KV-cache benchmark on one MI355X.

Default workload: Mistral-7B-shaped paged decode (32 query / 8 KV heads,
head_dim 128, bf16, 32 sequences with context lengths uniform in
[512, 4096], block size 32, shuffled pool).  One step = the slot writer for
the 32 new tokens plus the paged decode over all 32 sequences, all inputs
resident in HBM.  The pool is replicated so that consecutive steps read
different copies and the working set (>= 2 GB) cannot sit in the 256 MB
last-level cache.

Prints ONE JSON line.  ``value`` is the KV-read bandwidth of the whole step
(algorithmic K/V bytes the decode must read / step time).  ``roofline``
reports the decode alone (both of its kernels) against the 8 TB/s HBM peak,
timed with HIP events on the launch stream.  ``cpu_baseline`` times the CPU
oracle on the same inputs.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode: KV-read GB/s (% of HBM peak) and decode tokens/s, 1 MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def _args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="mistral_decode",
                    choices=["mistral_decode", "fp8_decode", "int8_decode", "sliding_decode",
                             "tiny_decode", "prefix_prefill", "sliding_prefill",
                             "sliding_prefill_fp8", "sliding_prefill_int8", "cow_copy"])
    ap.add_argument("--replicas", type=int, default=0, help="pool copies (0 = enough for 2 GB)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--separate-write", action="store_true",
                    help="time pa_reshape_and_cache + pa_decode instead of pa_decode_append")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds each core repeats the oracle's step for the CPU baseline "
                         "(0 = skip)")
    ap.add_argument("--no-sub-results", action="store_true",
                    help="default workload only: leave out the other workloads' lines")
    ap.add_argument("--calibrate-copy", type=float, default=0.0,
                    help="instead: time a plain device copy of this many GiB (counter scaling)")
    ap.add_argument("--dispatch-sweep", action="store_true",
                    help="instead: time decode split plans and the identity map over a grid "
                         "of batch sizes and context lengths (one JSON line per point)")
    return ap.parse_args()


# Sources whose change alters a kernel's memory traffic: the kernel file plus
# the shared device helpers and the host planner that picks its grid.
_KERNEL_SOURCES = {
    "decode_": ("paged_decode.hip", "common.hpp", "launch.hpp", "pa_api.cpp", "plan.hpp"),
    "prefill_": ("paged_prefill.hip", "common.hpp", "launch.hpp", "pa_api.cpp"),
    "copy_": ("copy_blocks.hip", "common.hpp", "launch.hpp", "pa_api.cpp"),
}


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines (comments do not change
    what is compiled)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(kernel_prefix: str) -> str:
    """sha256 over the code (comments stripped) of the HIP sources a kernel
    family is built from, to tie recorded counter data to a build of that
    kernel."""
    import hashlib
    d = os.path.join(ROOT, "paged_kv_cache_175_amd", "csrc")
    h = hashlib.sha256()
    for f in _KERNEL_SOURCES[kernel_prefix]:
        h.update(f.encode())
        with open(os.path.join(d, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def recorded_traffic(config: str, kernel_prefix: str):
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current
    sources of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    hashes = t.get("source_sha256")
    if not isinstance(hashes, dict) or hashes.get(kernel_prefix) != kernel_source_hash(kernel_prefix):
        return None
    total = 0.0
    found = False
    for k, v in t.get("configs", {}).get(config, {}).items():
        if k.startswith(kernel_prefix):
            total += v["fetch_bytes"] + v["write_bytes"]
            found = True
    return round(total) if found else None


def _workload(name):
    from paged_kv_cache_175_amd import workloads as W
    return {"mistral_decode": W.mistral_decode, "fp8_decode": W.fp8_decode,
            "int8_decode": W.int8_decode,
            "sliding_decode": W.sliding_decode, "tiny_decode": W.tiny_decode,
            "prefix_prefill": W.prefix_prefill, "sliding_prefill": W.sliding_prefill,
            "sliding_prefill_fp8": lambda: W.sliding_prefill(cache="e4m3"),
            "sliding_prefill_int8": lambda: W.sliding_prefill(cache="int8"),
            "cow_copy": W.cow_copy}[name]()


def _act_tensor(bits, act, torch):
    import numpy as np
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[act]
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dt).cuda()


def _cpu_info():
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


# --------------------------------------------------------------------------- decode


def _lib_code(name):
    from paged_kv_cache_175_amd import _lib
    return getattr(_lib, name)


def _decode_plan_name(wl, max_len, partition_tokens, ws_bytes):
    """Which decode kernel and plan the library picks (from the size of the
    workspace it asks for)."""
    from paged_kv_cache_175_amd import ops
    if partition_tokens:
        return "decode_split, forced splits"
    if ws_bytes == 0:
        return "decode_split, one workgroup per sequence and KV head"
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    rows = wl.B * wl.Hq * 2
    pair = (rnd(max(wl.B * wl.Hkv, ops.MIN_COUNTERS) * 4) + 2 * rnd(rows * 4)
            + rnd(rows * wl.D * 4))
    if ws_bytes == pair and wl.B <= 64:
        return "decode_split, pair mode"
    if wl.cache in ("e4m3", "int8") and max_len >= 1024:
        return "decode_balanced: equal page ranges of the batch"
    return "decode_split, split sequences"


def bench_decode(wl, a, torch):
    import numpy as np
    from paged_kv_cache_175_amd import ops, pool

    dev = torch.device("cuda", 0)
    kshape, vshape = ops.pool_shapes(wl.pool_blocks, wl.Hkv, wl.D, wl.BS)
    i8 = wl.cache == "int8"
    cache_dt = {"e4m3": torch.uint8, "int8": torch.int8, "bf16": torch.bfloat16,
                "f16": torch.float16}[wl.cache]
    elem = 1 if wl.cache in ("e4m3", "int8") else 2
    row_extra = 4 if i8 else 0          # an INT8 row also carries its fp32 scale
    pool_bytes = 2 * (math.prod(kshape) * elem + wl.pool_blocks * wl.Hkv * wl.BS * row_extra)
    R = a.replicas or min(64, max(1, math.ceil(2e9 / pool_bytes)))

    kc0 = torch.zeros(kshape, dtype=cache_dt, device=dev)
    vc0 = torch.zeros(vshape, dtype=cache_dt, device=dev)
    ksc0, vsc0 = ops.alloc_scale_pools(wl.pool_blocks, wl.Hkv, dev) if i8 else (None, None)
    # Cached tokens through the HIP writer, slots from the host block manager.
    ks, vs, sl = [], [], []
    for b in range(wl.B):
        n = wl.cached_k[b].shape[0]
        if n:
            pos = np.arange(wl.cached_pos0[b], wl.cached_pos0[b] + n)
            sl.append(pool.slots_from_table(wl.block_tables[b], pos, wl.BS, wl.window))
            ks.append(wl.cached_k[b])
            vs.append(wl.cached_v[b])
    if sl:
        ops.reshape_and_cache(_act_tensor(np.concatenate(ks), wl.act, torch),
                              _act_tensor(np.concatenate(vs), wl.act, torch), kc0, vc0,
                              torch.from_numpy(np.concatenate(sl).astype(np.int32)).to(dev),
                              wl.k_scale, wl.v_scale, key_scales=ksc0, value_scales=vsc0)
    del ks, vs, sl
    clone = lambda t: None if t is None else t.clone()  # noqa: E731
    pools = [(kc0, vc0, ksc0, vsc0)] + [(kc0.clone(), vc0.clone(), clone(ksc0), clone(vsc0))
                                        for _ in range(R - 1)]
    q0 = _act_tensor(wl.query, wl.act, torch)
    qs = [q0] + [q0.clone() for _ in range(R - 1)]
    new_k = _act_tensor(wl.new_k, wl.act, torch)
    new_v = _act_tensor(wl.new_v, wl.act, torch)
    new_slots = torch.from_numpy(np.array(
        [pool.slots_from_table(wl.block_tables[b], [wl.new_pos[b]], wl.BS, wl.window)[0]
         for b in range(wl.B)], dtype=np.int32)).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    max_len = int(wl.context_lens.max())
    need = ops.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, max_len, wl.window,
                                      a.partition_tokens)
    ws = ops.alloc_workspace(need, dev)
    out = torch.empty_like(q0)
    fmt = {"e4m3": _lib_code("PA_F8E4M3"), "int8": _lib_code("PA_I8"),
           "f16": _lib_code("PA_F16")}.get(wl.cache, _lib_code("PA_BF16"))
    need_fmt = ops.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, max_len, wl.window,
                                          a.partition_tokens, fmt)

    # One step: store the new tokens and attend.  Default: the fused
    # pa_decode_append (pa_decode_append_i8 for an INT8 cache; one launch);
    # --separate-write: pa_reshape_and_cache then pa_decode.
    separate = a.separate_write
    writes, decodes = [], []
    for r in range(R):
        kc, vc, ksc, vsc = pools[r]
        if separate:
            writes.append(ops.prepare_reshape_and_cache(new_k, new_v, kc, vc, new_slots,
                                                        wl.k_scale, wl.v_scale,
                                                        key_scales=ksc, value_scales=vsc))
            decodes.append(ops.prepare_decode(qs[r], kc, vc, bt, cl, max_len, wl.scale, out, ws,
                                              wl.k_scale, wl.v_scale, wl.window,
                                              a.partition_tokens, key_scales=ksc,
                                              value_scales=vsc))
        else:
            writes.append(lambda: None)
            decodes.append(ops.prepare_decode(qs[r], kc, vc, bt, cl, max_len, wl.scale, out, ws,
                                              wl.k_scale, wl.v_scale, wl.window,
                                              a.partition_tokens, new_key=new_k,
                                              new_value=new_v, key_scales=ksc,
                                              value_scales=vsc))

    kv_tokens = wl.kv_read_tokens()
    kv_bytes = kv_tokens * wl.Hkv * (wl.D * elem + row_extra) * 2
    # read K,V act; write K,V cache (and their scales)
    write_bytes = wl.B * wl.Hkv * (wl.D * (2 * 2 + 2 * elem) + 2 * row_extra)
    qo_bytes = 2 * wl.B * wl.Hq * wl.D * 2

    for i in range(a.warmup):
        writes[i % R]()
        decodes[i % R]()
    torch.cuda.synchronize()

    # Timed region 1: K back-to-back steps between two events (step time).
    K = a.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        writes[i % R]()
        decodes[i % R]()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    step_s = total_ms / K * 1e-3
    # Timed region 2: K back-to-back launches of the decode kernel alone
    # between two events on its launch stream: its average launch duration,
    # for the roofline.  (With the fused write this is region 1 again; with
    # --separate-write the writer is left out.)
    d_start = torch.cuda.Event(enable_timing=True)
    d_end = torch.cuda.Event(enable_timing=True)
    d_start.record()
    for i in range(K):
        decodes[i % R]()
    d_end.record()
    torch.cuda.synchronize()
    dec_avg_s = d_start.elapsed_time(d_end) / K * 1e-3
    # Timed region 3: an event pair around each decode launch, for the spread
    # of single-launch times (each includes the event overhead, a few us).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        writes[i % R]()
        ev[i][0].record()
        decodes[i % R]()
        ev[i][1].record()
    torch.cuda.synchronize()
    launch_us = np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3

    achieved = kv_bytes / dec_avg_s / 1e9
    res = {
        "metric": METRIC,
        "value": round(kv_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"e4m3": "e4m3->bf16", "int8": "i8->bf16"}.get(wl.cache, "bf16"),
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
            "head_dim": wl.D, "block_size": wl.BS, "act_dtype": wl.act,
            "cache_dtype": wl.cache, "window": wl.window, "seed": wl.meta["seed"],
            "context_tokens_read": kv_tokens, "max_context_len": max_len,
            "new_tokens_written": wl.B, "pool_blocks": wl.pool_blocks, "replicas": R,
            "partition_tokens": a.partition_tokens or "auto",
            "step": "pa_reshape_and_cache + pa_decode" if separate
                    else "pa_decode_append (write + decode in one launch)",
        },
        "tokens_per_s": round(wl.B / step_s, 1),
        "decode_tokens_per_s": round(wl.B / dec_avg_s, 1),
        "decode_us": round(dec_avg_s * 1e6, 3),
        "decode_launch_us_p10_p50_p90": [round(float(x), 3) for x in
                                         np.percentile(launch_us, [10, 50, 90])],
        "step_us": round(step_s * 1e6, 3),
        "wall_us_per_step": round(wall / K * 1e6, 3),
        "kv_bytes_per_step": kv_bytes,
        "other_bytes_per_step": write_bytes + qo_bytes,
        "roofline": {
            "kernel": ("pa_decode" if separate else "pa_decode_append")
                      + f" ({_decode_plan_name(wl, max_len, a.partition_tokens, need_fmt)}; "
                        "split sequences merge inside the launch)",
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(wl.name, "decode_"),
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    return res, (wl, kv_bytes)


# --------------------------------------------------------------------------- CPU baseline
# The oracle (unchanged) on every core of this process's CPU share: one
# single-threaded worker process per core (at most 16, a host's share per
# GPU), each on its own group of sequences with its own compact pool (the
# blocks its sequences own, renumbered).  The workers populate their pools
# untimed, meet at a barrier, then repeat their step for the time budget; the
# batch's step time is the slowest group's.  Workers are forked from a
# forkserver started before this process touches the GPU.

_MP = None


def _cpu_cores() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _start_cpu_pool() -> None:
    global _MP
    if _MP is not None:
        return
    import multiprocessing as mp
    _MP = mp.get_context("forkserver")
    _MP.set_forkserver_preload(["numpy", "oracle.attention", "oracle.cache", "oracle.pool"])
    from multiprocessing import forkserver
    forkserver.ensure_running()


def _groups(weights, n):
    """Indices in at most n groups of about equal total weight."""
    import numpy as np
    order = np.argsort(-np.asarray(weights, dtype=np.float64), kind="stable")
    groups, load = [[] for _ in range(n)], [0.0] * n
    for i in order:
        g = load.index(min(load))
        groups[g].append(int(i))
        load[g] += float(weights[i])
    return [sorted(g) for g in groups if g]


def _compact(tables, nblk):
    """Renumber the first nblk[r] entries of each table row into 0..n-1."""
    import numpy as np
    used = np.unique(np.concatenate([tables[r, :nblk[r]] for r in range(len(nblk))]))
    local = {int(x): k for k, x in enumerate(used)}
    out = np.zeros_like(tables)
    for r in range(len(nblk)):
        out[r, :nblk[r]] = [local[int(x)] for x in tables[r, :nblk[r]]]
    return out, int(used.size)


def _cpu_pools(wl):
    from oracle import cache as o_cache
    kc, vc = o_cache.empty_pools(wl.pool_blocks, wl.Hkv, wl.BS, wl.D, wl.cache, 0)
    if wl.cache == "int8":
        return kc, vc, *o_cache.empty_scale_pools(wl.pool_blocks, wl.Hkv, wl.BS)
    return kc, vc, wl.k_scale, wl.v_scale


def _cpu_setup_decode(wl):
    import numpy as np
    from oracle import cache as o_cache
    from oracle import pool as o_pool
    kc, vc, ks, vs = _cpu_pools(wl)

    def row(pos):
        return o_pool.ring_index(int(pos), wl.window) if wl.window else int(pos)

    for b in range(wl.B):
        n = wl.cached_k[b].shape[0]
        slots = [o_cache.slot_of(wl.block_tables[b], row(wl.cached_pos0[b] + t), wl.BS)
                 for t in range(n)]
        o_cache.reshape_and_cache(wl.cached_k[b], wl.cached_v[b], kc, vc, np.array(slots),
                                  wl.act, wl.cache, ks, vs)
    new_slots = np.array([o_cache.slot_of(wl.block_tables[b], row(wl.new_pos[b]), wl.BS)
                          for b in range(wl.B)])
    return wl, (kc, vc, ks, vs), new_slots


def _cpu_step_decode(state):
    from oracle import attention as o_attn
    from oracle import cache as o_cache
    wl, (kc, vc, ks, vs), new_slots = state
    o_cache.reshape_and_cache(wl.new_k, wl.new_v, kc, vc, new_slots, wl.act, wl.cache, ks, vs)
    o_attn.decode(wl.query, wl.act, kc, vc, wl.cache, wl.block_tables, wl.context_lens,
                  wl.scale, ks, vs, wl.window)


def _cpu_setup_prefill(wl):
    import numpy as np
    from oracle import cache as o_cache
    kc, vc, ks, vs = _cpu_pools(wl)
    slots = [o_cache.slot_of(wl.block_tables[0], t, wl.BS) for t in range(wl.prefix_len)]
    o_cache.reshape_and_cache(wl.prefix_k, wl.prefix_v, kc, vc, np.array(slots), wl.act,
                              wl.cache, ks, vs)
    chunk_slots = [np.array([o_cache.slot_of(wl.block_tables[b], wl.prefix_len + t, wl.BS)
                             for t in range(int(wl.chunk_lens[b]))]) for b in range(wl.B)]
    return wl, (kc, vc, ks, vs), chunk_slots


def _cpu_step_prefill(state):
    from oracle import attention as o_attn
    from oracle import cache as o_cache
    wl, (kc, vc, ks, vs), chunk_slots = state
    for b in range(wl.B):
        o_cache.reshape_and_cache(wl.chunk_k[b], wl.chunk_v[b], kc, vc, chunk_slots[b], wl.act,
                                  wl.cache, ks, vs)
    o_attn.prefill_chunk(wl.query, wl.act, wl.cu_q_lens, kc, vc, wl.cache, wl.block_tables,
                         wl.context_lens, wl.scale, ks, vs)


def _cpu_setup_window(wl):
    import numpy as np
    from oracle import cache as o_cache
    from oracle import pool as o_pool
    kc, vc, ks, vs = _cpu_pools(wl)
    for b in range(wl.B):
        pos = range(int(wl.hist_pos0[b]), int(wl.hist_lens[b]))
        slots = [o_cache.slot_of(wl.block_tables[b], o_pool.ring_index(p, wl.window), wl.BS)
                 for p in pos]
        o_cache.reshape_and_cache(wl.hist_k[b], wl.hist_v[b], kc, vc, np.array(slots), wl.act,
                                  wl.cache, ks, vs)
    return wl, (kc, vc, ks, vs)


def _cpu_step_window(state):
    from oracle import attention as o_attn
    wl, (kc, vc, ks, vs) = state
    o_attn.prefill_chunk_window(wl.query, wl.act, wl.chunk_k, wl.chunk_v, wl.cu_q_lens, kc, vc,
                                wl.cache, wl.block_tables, wl.context_lens, wl.scale,
                                wl.window, rows=wl.rows, k_scale=ks, v_scale=vs)


def _cpu_setup_copy(wl):
    import numpy as np
    from oracle import cache as o_cache
    kc, vc = o_cache.empty_pools(wl.num_blocks, wl.Hkv, wl.BS, wl.D, wl.cache, 0)
    rng = np.random.default_rng(0)
    kc[...] = rng.integers(0, 1 << 14, kc.shape).astype(kc.dtype)
    vc[...] = rng.integers(0, 1 << 14, vc.shape).astype(vc.dtype)
    return wl, kc, vc


def _cpu_step_copy(state):
    from oracle import cache as o_cache
    wl, kc, vc = state
    o_cache.copy_blocks(kc, vc, wl.mapping)


_CPU_KINDS = {"decode": (_cpu_setup_decode, _cpu_step_decode),
              "copy": (_cpu_setup_copy, _cpu_step_copy),
              "prefill": (_cpu_setup_prefill, _cpu_step_prefill),
              "window": (_cpu_setup_window, _cpu_step_window)}


def _cpu_worker(job, barrier, results):
    import types
    from threadpoolctl import threadpool_limits
    try:
        with threadpool_limits(limits=1):
            setup, step = _CPU_KINDS[job.pop("kind")]
            seconds = job.pop("seconds")
            jid = job.pop("id")
            state = setup(types.SimpleNamespace(**job))
            barrier.wait(timeout=1800)
            t0 = time.perf_counter()
            reps = 0
            while True:
                step(state)
                reps += 1
                t = time.perf_counter() - t0
                if t >= seconds:
                    break
        results.put((jid, reps, t, None))
    except Exception as e:  # pragma: no cover - reported to the parent
        barrier.abort()
        results.put((job.get("id", -1), 0, 0.0, repr(e)))


def _cpu_run(jobs, seconds):
    """Run every job in its own worker process; returns the slowest job's
    seconds per step and the reps and seconds of each."""
    _start_cpu_pool()
    n = len(jobs)
    barrier = _MP.Barrier(n)
    results = _MP.Queue()
    for i, j in enumerate(jobs):
        j.update(id=i, seconds=seconds)
    procs = [_MP.Process(target=_cpu_worker, args=(j, barrier, results)) for j in jobs]
    for p in procs:
        p.start()
    got = [results.get(timeout=3600) for _ in range(n)]
    for p in procs:
        p.join()
    errs = [e for (_, _, _, e) in got if e]
    if errs:
        raise RuntimeError(f"CPU baseline worker failed: {errs[0]}")
    per = max(t / reps for (_, reps, t, _) in got)
    return per, got


def _decode_job(wl, g):
    import numpy as np
    L = wl.context_lens.astype(np.int64)
    if wl.window:
        L = np.minimum(L, wl.window)
    nblk = [int(-(-int(L[b]) // wl.BS)) for b in g]
    tables, nb = _compact(wl.block_tables[g], nblk)
    return dict(kind="decode", act=wl.act, cache=wl.cache, B=len(g), Hq=wl.Hq, Hkv=wl.Hkv,
                D=wl.D, BS=wl.BS, window=wl.window, scale=wl.scale, k_scale=wl.k_scale,
                v_scale=wl.v_scale, pool_blocks=nb, block_tables=tables,
                context_lens=wl.context_lens[g], query=wl.query[g],
                cached_pos0=wl.cached_pos0[g], cached_k=[wl.cached_k[b] for b in g],
                cached_v=[wl.cached_v[b] for b in g], new_pos=wl.new_pos[g],
                new_k=wl.new_k[g], new_v=wl.new_v[g])


def cpu_baseline_decode(wl, kv_bytes, seconds):
    """The oracle on the same inputs, the batch's sequences spread over the
    CPU's cores: per group, untimed pool population, then timed repetitions
    of (writer for the group's new tokens + decode of its sequences)."""
    import numpy as np
    L = wl.context_lens.astype(np.int64)
    if wl.window:
        L = np.minimum(L, wl.window)
    groups = _groups(L + 64, _cpu_cores())
    per, got = _cpu_run([_decode_job(wl, g) for g in groups], seconds)
    reps = min(r for (_, r, _, _) in got)
    return {
        "value": round(kv_bytes / per / 1e9, 4), "unit": "GB/s", "cores": len(groups),
        "kind": "oracle", "tokens_per_s": round(wl.B / per, 3),
        "seconds_per_step": round(per, 4),
        "sample": f"full workload ({wl.B} sequences, {wl.kv_read_tokens()} tokens per KV head): "
                  f"writer + fp64 decode, sequences split by tokens over {len(groups)} "
                  f"single-threaded processes, each repeating its step for {seconds:.0f} s "
                  f"(at least {reps} repetitions); step time = the slowest group's",
        "cpu_model": _cpu_info(), "host_cpus": len(os.sched_getaffinity(0)),
    }


def cpu_baseline_prefill(wl, seconds):
    """The oracle's writer + chunked prefill on the same inputs, one group of
    sequences per core (each job writes the shared prefix into its own pool,
    untimed, then times the chunk writes and the prefill of its sequences)."""
    import numpy as np
    nsh = wl.prefix_len // wl.BS
    groups = _groups(wl.chunk_lens.astype(np.int64), _cpu_cores())
    jobs = []
    for g in groups:
        nblk = [int(-(-int(wl.context_lens[b]) // wl.BS)) for b in g]
        assert all(np.array_equal(wl.block_tables[b, :nsh], wl.block_tables[0, :nsh]) for b in g)
        tables, nb = _compact(wl.block_tables[g], nblk)
        rows = np.concatenate([np.arange(wl.cu_q_lens[b], wl.cu_q_lens[b + 1]) for b in g])
        cu = np.zeros(len(g) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(wl.chunk_lens[g])
        jobs.append(dict(kind="prefill", act=wl.act, cache=wl.cache, B=len(g), Hq=wl.Hq,
                         Hkv=wl.Hkv, D=wl.D, BS=wl.BS, scale=wl.scale, k_scale=wl.k_scale,
                         v_scale=wl.v_scale, pool_blocks=nb, prefix_len=wl.prefix_len,
                         prefix_k=wl.prefix_k, prefix_v=wl.prefix_v,
                         chunk_lens=wl.chunk_lens[g], chunk_k=[wl.chunk_k[b] for b in g],
                         chunk_v=[wl.chunk_v[b] for b in g], cu_q_lens=cu,
                         context_lens=wl.context_lens[g], block_tables=tables,
                         query=wl.query[rows]))
    per, got = _cpu_run(jobs, seconds)
    reps = min(r for (_, r, _, _) in got)
    flops = wl.flops()
    return {
        "value": round(flops / per / 1e12, 6), "unit": "TFLOP/s", "cores": len(groups),
        "kind": "oracle", "tokens_per_s": round(wl.total_q / per, 3),
        "seconds_per_step": round(per, 3),
        "sample": f"full workload ({wl.B} sequences x {int(wl.chunk_lens[0])} query rows): "
                  f"chunk writer + fp64 causal prefill, sequences split over {len(groups)} "
                  f"single-threaded processes, each repeating its step for {seconds:.0f} s "
                  f"(at least {reps} repetitions); step time = the slowest group's",
        "cpu_model": _cpu_info(), "host_cpus": len(os.sched_getaffinity(0)),
    }


def cpu_baseline_window(wl, seconds, rows_per_core=16):
    """The oracle's window prefill on a bounded sample: each core takes one
    sequence's ring (populated untimed) and ``rows_per_core`` query rows
    spread over the chunk, every head; the value is the sample's attention
    FLOPs over the slowest core's time."""
    import numpy as np
    n = _cpu_cores()
    C = int(wl.chunk_lens[0])
    jobs, flops, nrows = [], 0, 0
    for i in range(n):
        b = i % wl.B
        k = i // wl.B
        per_seq = -(-n // wl.B)
        rows = sorted({int((k + per_seq * r) * C // (per_seq * rows_per_core))
                       for r in range(rows_per_core)})
        tables, nb = _compact(wl.block_tables[b:b + 1], [wl.block_tables.shape[1]])
        q0, q1 = int(wl.cu_q_lens[b]), int(wl.cu_q_lens[b + 1])
        start = int(wl.context_lens[b]) - (q1 - q0)
        for j in rows:
            flops += 4 * wl.D * wl.Hq * min(start + j + 1, wl.window)
        nrows += len(rows)
        jobs.append(dict(kind="window", act=wl.act, cache=wl.cache, B=1, Hq=wl.Hq, Hkv=wl.Hkv,
                         D=wl.D, BS=wl.BS, window=wl.window, scale=wl.scale,
                         k_scale=wl.k_scale, v_scale=wl.v_scale, pool_blocks=nb,
                         hist_lens=wl.hist_lens[b:b + 1], hist_pos0=wl.hist_pos0[b:b + 1],
                         chunk_lens=wl.chunk_lens[b:b + 1], cu_q_lens=np.array([0, q1 - q0]),
                         context_lens=wl.context_lens[b:b + 1], block_tables=tables,
                         query=wl.query[q0:q1], chunk_k=wl.chunk_k[q0:q1],
                         chunk_v=wl.chunk_v[q0:q1], hist_k=[wl.hist_k[b]],
                         hist_v=[wl.hist_v[b]], rows={(0, j) for j in rows}))
    per, got = _cpu_run(jobs, seconds)
    return {
        "value": round(flops / per / 1e12, 9), "unit": "TFLOP/s", "cores": n, "kind": "oracle",
        "seconds_per_step": round(per, 3),
        "sample": f"{nrows} query rows ({rows_per_core} per core, spread over the chunks of "
                  f"all {wl.B} sequences), every head, over full rings of {wl.window} rows: "
                  f"fp64 window attention ({flops:.3e} FLOP), {n} single-threaded processes; "
                  f"time = the slowest core's; ring population untimed",
        "cpu_model": _cpu_info(), "host_cpus": len(os.sched_getaffinity(0)),
    }


# --------------------------------------------------------------------------- prefill


def bench_prefill(wl, a, torch):
    import numpy as np
    from paged_kv_cache_175_amd import ops, pool

    dev = torch.device("cuda", 0)
    kshape, vshape = ops.pool_shapes(wl.pool_blocks, wl.Hkv, wl.D, wl.BS)
    kc = torch.zeros(kshape, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros(vshape, dtype=torch.bfloat16, device=dev)
    sl = pool.slots_from_table(wl.block_tables[0], np.arange(wl.prefix_len), wl.BS)
    ops.reshape_and_cache(_act_tensor(wl.prefix_k, wl.act, torch),
                          _act_tensor(wl.prefix_v, wl.act, torch), kc, vc,
                          torch.from_numpy(sl).to(dev))
    ck = _act_tensor(np.concatenate(wl.chunk_k), wl.act, torch)
    cv = _act_tensor(np.concatenate(wl.chunk_v), wl.act, torch)
    chunk_slots = torch.from_numpy(np.concatenate([
        pool.slots_from_table(wl.block_tables[b],
                              np.arange(wl.prefix_len, wl.prefix_len + int(wl.chunk_lens[b])),
                              wl.BS) for b in range(wl.B)])).to(dev)
    q = _act_tensor(wl.query, wl.act, torch)
    # Replicas of the pools, the queries and the output (and the chunk's K/V),
    # so that consecutive steps touch different copies (>= 2 GB in all) and
    # the 256 MB last-level cache cannot hold a step's working set.
    rep_bytes = 2 * kc.numel() * 2 + 2 * q.numel() * 2 + 2 * ck.numel() * 2
    R = a.replicas or max(1, math.ceil(2e9 / rep_bytes))
    cu = torch.from_numpy(wl.cu_q_lens).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    writes, runs = [], []
    for r in range(R):
        kr, vr = (kc, vc) if r == 0 else (kc.clone(), vc.clone())
        qr, ckr, cvr = (q, ck, cv) if r == 0 else (q.clone(), ck.clone(), cv.clone())
        writes.append(ops.prepare_reshape_and_cache(ckr, cvr, kr, vr, chunk_slots))
        runs.append(ops.prepare_prefill_chunk(qr, cu, kr, vr, bt, cl, int(wl.chunk_lens.max()),
                                              wl.scale, torch.empty_like(q)))
    for i in range(a.warmup):
        writes[i % R]()
        runs[i % R]()
    torch.cuda.synchronize()
    K = a.steps
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(K):
        writes[i % R]()
        runs[i % R]()
    t1.record()
    torch.cuda.synchronize()
    step_s = t0.elapsed_time(t1) / K * 1e-3
    # Kernel duration: K back-to-back prefill launches between two events.
    t2 = torch.cuda.Event(enable_timing=True)
    t3 = torch.cuda.Event(enable_timing=True)
    t2.record()
    for i in range(K):
        runs[i % R]()
    t3.record()
    torch.cuda.synchronize()
    pre_s = t2.elapsed_time(t3) / K * 1e-3
    flops = wl.flops()
    tf = flops / pre_s / 1e12
    return {
        "metric": "chunked prefill over shared prefix: attention TFLOP/s, 1 MI355X",
        "value": round(flops / step_s / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": a.warmup, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "prefix_len": wl.prefix_len,
                   "chunk_len": int(wl.chunk_lens[0]), "block_size": wl.BS, "replicas": R,
                   "step": "pa_reshape_and_cache (chunk) + pa_prefill_chunk"},
        "prefill_us": round(pre_s * 1e6, 3), "step_us": round(step_s * 1e6, 3),
        "tokens_per_s": round(wl.total_q / step_s, 1),
        "roofline": {"kernel": "pa_prefill_chunk", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(wl.name, "prefill_"),
                     "algorithmic_flops_per_launch": flops},
    }


def bench_window_prefill(wl, a, torch):
    """One step = window prefill attention of every chunk over its ring, then
    the ring write of the chunk's landing tokens."""
    import numpy as np
    from paged_kv_cache_175_amd import ops, pool

    dev = torch.device("cuda", 0)
    kshape, vshape = ops.pool_shapes(wl.pool_blocks, wl.Hkv, wl.D, wl.BS)
    cache_dt = {"e4m3": torch.uint8, "int8": torch.int8}.get(wl.cache, torch.bfloat16)
    kc = torch.zeros(kshape, dtype=cache_dt, device=dev)
    vc = torch.zeros(vshape, dtype=cache_dt, device=dev)
    # Quantised rings: E4M3 with the workload's tensor scales, INT8 with its
    # row scale pools.
    ks, vs = (ops.alloc_scale_pools(wl.pool_blocks, wl.Hkv, dev) if wl.cache == "int8"
              else (None, None))
    qkw = dict(k_scale=wl.k_scale, v_scale=wl.v_scale, key_scales=ks, value_scales=vs)
    hk, hv, hs, cs = [], [], [], []
    for b in range(wl.B):
        pos = np.arange(int(wl.hist_pos0[b]), int(wl.hist_lens[b]))
        hs.append(pool.slots_from_table(wl.block_tables[b], pos, wl.BS, wl.window))
        hk.append(wl.hist_k[b])
        hv.append(wl.hist_v[b])
        C, ctx = int(wl.chunk_lens[b]), int(wl.context_lens[b])
        sl = pool.slots_from_table(wl.block_tables[b], np.arange(ctx - C, ctx), wl.BS,
                                   wl.window)
        sl[: max(0, C - wl.window)] = -1       # overwritten within the chunk
        cs.append(sl)
    ops.reshape_and_cache(_act_tensor(np.concatenate(hk), wl.act, torch),
                          _act_tensor(np.concatenate(hv), wl.act, torch), kc, vc,
                          torch.from_numpy(np.concatenate(hs)).to(dev), **qkw)
    q = _act_tensor(wl.query, wl.act, torch)
    k = _act_tensor(wl.chunk_k, wl.act, torch)
    v = _act_tensor(wl.chunk_v, wl.act, torch)
    out = torch.empty_like(q)
    cu = torch.from_numpy(wl.cu_q_lens).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    slots = torch.from_numpy(np.concatenate(cs)).to(dev)
    # The step reads the pre-chunk ring; writing the chunk each step would
    # change what the next step reads, so the write goes to a second copy.
    # Replicas of everything a step touches (>= 2 GB in all) rotate so that
    # the 256 MB last-level cache cannot hold a step's working set.
    clone = lambda t: None if t is None else t.clone()  # noqa: E731
    ring_bytes = 2 * kc.numel() * kc.element_size() + (2 * ks.numel() * 4 if ks is not None
                                                       else 0)
    rep_bytes = 2 * ring_bytes + 2 * q.numel() * 2 + 2 * k.numel() * 2
    R = a.replicas or max(1, math.ceil(2e9 / rep_bytes))
    runs, writes = [], []
    for r in range(R):
        if r == 0:
            kr, vr, ksr, vsr, qr, kk, vv = kc, vc, ks, vs, q, k, v
        else:
            kr, vr, ksr, vsr = kc.clone(), vc.clone(), clone(ks), clone(vs)
            qr, kk, vv = q.clone(), k.clone(), v.clone()
        writes.append(ops.prepare_reshape_and_cache(kk, vv, kr.clone(), vr.clone(), slots,
                                                    wl.k_scale, wl.v_scale,
                                                    key_scales=clone(ksr),
                                                    value_scales=clone(vsr)))
        o = out if r == 0 else torch.empty_like(q)
        kw = dict(k_scale=wl.k_scale, v_scale=wl.v_scale, key_scales=ksr, value_scales=vsr)
        runs.append(lambda qr=qr, kk=kk, vv=vv, kr=kr, vr=vr, o=o, kw=kw:
                    ops.prefill_chunk_window(qr, kk, vv, cu, kr, vr, bt, cl,
                                             int(wl.chunk_lens.max()), wl.scale, wl.window,
                                             out=o, **kw))

    for i in range(a.warmup):
        runs[i % R]()
        writes[i % R]()
    torch.cuda.synchronize()
    K = a.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for i in range(K):
        runs[i % R]()
        writes[i % R]()
    ev[1].record()
    torch.cuda.synchronize()
    step_s = ev[0].elapsed_time(ev[1]) / K * 1e-3
    ev[2].record()
    for i in range(K):
        runs[i % R]()
    ev[3].record()
    torch.cuda.synchronize()
    pre_s = ev[2].elapsed_time(ev[3]) / K * 1e-3
    flops = wl.flops()
    tf = flops / pre_s / 1e12
    return {
        "metric": "sliding-window chunked prefill into a ring: attention TFLOP/s, 1 MI355X",
        "value": round(flops / step_s / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": a.warmup, "ms_per_step": round(step_s * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "window": wl.window, "history": int(wl.hist_lens[0]),
                   "chunk_len": int(wl.chunk_lens[0]), "block_size": wl.BS,
                   "ring": wl.cache, "replicas": R,
                   "step": "pa_prefill_chunk_window + ring write of the landing tokens"},
        "prefill_us": round(pre_s * 1e6, 3), "step_us": round(step_s * 1e6, 3),
        "tokens_per_s": round(wl.total_q / step_s, 1),
        "roofline": {"kernel": "pa_prefill_chunk_window", "bound": "mfma",
                     "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(wl.name, "prefill_"),
                     "algorithmic_flops_per_launch": flops},
    }


def dispatch_sweep(a, torch):
    """Decode launch time of the library's automatic split plan, of one pass
    without splits, of forced partitions, and of the identity map, over a
    grid of batch sizes and uniform context lengths (Mistral decode shape,
    bf16).  Pools are replicated so that each launch reads cold HBM."""
    import numpy as np
    from paged_kv_cache_175_amd import ops

    Hq, Hkv, D, BS = 32, 8, 128, 32
    dev = torch.device("cuda", 0)
    rows = []
    for B in (1, 8, 32, 128):
        for L in (256, 512, 1024, 2048, 4096, 8192, 16384):
            M = -(-L // BS)
            NB = B * M
            per = NB * Hkv * BS * D * 2 * 2
            R = max(1, min(48, (2 << 30) // per))
            kshape, vshape = ops.pool_shapes(NB, Hkv, D, BS)
            pools = [(torch.randn(kshape, device=dev).to(torch.bfloat16),
                      torch.randn(vshape, device=dev).to(torch.bfloat16)) for _ in range(R)]
            rng = np.random.default_rng(B * 100000 + L)
            perm = torch.from_numpy(rng.permutation(NB).astype(np.int32).reshape(B, M)).to(dev)
            q = torch.randn(B, Hq, D, device=dev).to(torch.bfloat16)
            cl = torch.full((B,), L, dtype=torch.int32, device=dev)
            out = torch.empty_like(q)
            variants = {"auto": (perm, 0), "identity": (ops.IdentityMap(M), 0),
                        "one_pass": (perm, M * BS)}
            for p in (256, 512, 1024, 2048):
                if p < L:
                    variants[f"part{p}"] = (perm, p)
            row = {"B": B, "L": L, "replicas": R}
            for name, (bt, part) in variants.items():
                ws = ops.alloc_workspace(ops.decode_workspace_bytes(B, Hq, Hkv, D, L, 0, part),
                                         dev)
                calls = [ops.prepare_decode(q, kc, vc, bt, cl, L, 1.0 / math.sqrt(D), out, ws,
                                            partition_tokens=part) for kc, vc in pools]
                for _ in range(2):
                    for c in calls:
                        c()
                times = []
                for _ in range(5):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for c in calls:
                        c()
                    e1.record()
                    e1.synchronize()
                    times.append(e0.elapsed_time(e1) * 1e3 / len(calls))
                row[name + "_us"] = round(sorted(times)[2], 2)
            row["auto_GBps"] = round(B * L * Hkv * D * 4 / row["auto_us"] / 1e3, 1)
            best = min((v, k) for k, v in row.items() if k.endswith("_us"))
            row["best"] = best[1][:-3]
            print(json.dumps(row), flush=True)
            rows.append(row)
            del pools
            torch.cuda.empty_cache()
    return {"dispatch_sweep": "decode split plans and identity map", "points": len(rows)}


def bench_copy_blocks(wl, a, torch):
    """Copy-on-write block copies (``pa_copy_blocks``): one step = the whole
    burst of ``N`` copies; HBM-bound, read + write bytes against 8 TB/s."""
    from paged_kv_cache_175_amd import ops

    dev = torch.device("cuda", 0)
    kshape, vshape = ops.pool_shapes(wl.num_blocks, wl.Hkv, wl.D, wl.BS)
    kc = torch.randn(kshape, device=dev).to(torch.bfloat16)
    vc = torch.randn(vshape, device=dev).to(torch.bfloat16)
    mapping = torch.from_numpy(wl.mapping).to(dev)
    for _ in range(a.warmup):
        ops.copy_blocks(kc, vc, mapping)
    torch.cuda.synchronize()
    K = a.steps
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        ops.copy_blocks(kc, vc, mapping)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / K * 1e-3
    N = wl.mapping.shape[0]
    moved = 2 * N * wl.block_bytes()       # every block read once and written once
    gbs = moved / s / 1e9
    res = {
        "metric": "copy-on-write block copies: HBM GB/s (read + write), 1 MI355X",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": a.warmup,
        "ms_per_step": round(s * 1e3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "copies": N, "kv_heads": wl.Hkv, "head_dim": wl.D,
                   "block_size": wl.BS, "block_bytes": wl.block_bytes(),
                   "pool_blocks": wl.num_blocks},
        "copy_us": round(s * 1e6, 3),
        "roofline": {"kernel": "pa_copy_blocks (copy_blocks_kernel)", "bound": "hbm",
                     "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(wl.name, "copy_"),
                     "algorithmic_bytes_per_launch": moved},
    }
    if a.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_copy(wl, moved, a.cpu_seconds)
    return res


def cpu_baseline_copy(wl, moved, seconds):
    """The oracle's block copy over the CPU's cores: each core takes an equal
    share of the copy pairs on a compact pool of just their blocks."""
    import numpy as np
    n = _cpu_cores()
    jobs = []
    for part in np.array_split(np.arange(wl.mapping.shape[0]), n):
        if part.size == 0:
            continue
        pairs = wl.mapping[part]
        used, local = np.unique(pairs, return_inverse=True)
        jobs.append(dict(kind="copy", cache=wl.cache, Hkv=wl.Hkv, D=wl.D, BS=wl.BS,
                         num_blocks=int(used.size),
                         mapping=local.reshape(pairs.shape).astype(np.int32)))
    per, got = _cpu_run(jobs, seconds)
    reps = min(r for (_, r, _, _) in got)
    return {"value": round(moved / per / 1e9, 4), "unit": "GB/s", "cores": len(jobs),
            "kind": "oracle", "seconds_per_step": round(per, 4),
            "sample": f"full burst ({wl.mapping.shape[0]} block copies) split over {len(jobs)} "
                      f"single-threaded processes, each on a pool of its pairs' blocks, "
                      f"repeating its share for {seconds:.0f} s (at least {reps} "
                      f"repetitions); time = the slowest process's",
            "cpu_model": _cpu_info(), "host_cpus": len(os.sched_getaffinity(0))}


def calibrate_copy(gib, a, torch):
    n = int(gib * (1 << 30))
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(a.steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    s = t0.elapsed_time(t1) / a.steps * 1e-3
    return {"calibration": "device copy", "bytes_read": n, "bytes_written": n,
            "us_per_copy": round(s * 1e6, 2), "GBps_read_plus_write": round(2 * n / s / 1e9, 1)}


SUB_RESULTS = (("C1", "tiny_decode"), ("C3", "fp8_decode"), ("C4", "sliding_decode"),
               ("C5", "prefix_prefill"))


def _sub_result(res):
    """What another workload's line adds to the default one: its time, its
    roofline (with the recorded traffic) and its own value."""
    keep = ("value", "unit", "ms_per_step", "step_us", "decode_us", "prefill_us",
            "decode_launch_us_p10_p50_p90", "tokens_per_s")
    d = {"workload": res["config"]["workload"]}
    d.update({k: res[k] for k in keep if k in res})
    d["roofline"] = res["roofline"]
    return d


def main():
    a = _args()
    if a.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1 "
                                   "(the path shards by sequence or KV head, but no "
                                   "multi-GPU code is built)"}))
        sys.exit(2)
    if a.cpu_seconds > 0:
        _start_cpu_pool()           # before anything touches the GPU
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if a.calibrate_copy > 0:
        print(json.dumps(calibrate_copy(a.calibrate_copy, a, torch)))
        return
    if a.dispatch_sweep:
        print(json.dumps(dispatch_sweep(a, torch)))
        return
    wl = _workload(a.config)
    if a.config == "prefix_prefill":
        res = bench_prefill(wl, a, torch)
        if a.cpu_seconds > 0:
            res["cpu_baseline"] = cpu_baseline_prefill(wl, a.cpu_seconds)
    elif a.config.startswith("sliding_prefill"):
        res = bench_window_prefill(wl, a, torch)
        if a.cpu_seconds > 0:
            res["cpu_baseline"] = cpu_baseline_window(wl, a.cpu_seconds)
    elif a.config == "cow_copy":
        res = bench_copy_blocks(wl, a, torch)
    else:
        res, (wl, kv_bytes) = bench_decode(wl, a, torch)
        if a.config == "mistral_decode" and not a.no_sub_results and not a.partition_tokens:
            subs = {}
            for tag, name in SUB_RESULTS:
                torch.cuda.empty_cache()
                w = _workload(name)
                r = bench_prefill(w, a, torch) if name == "prefix_prefill" else \
                    bench_decode(w, a, torch)[0]
                subs[tag] = _sub_result(r)
                del w, r
            torch.cuda.empty_cache()
            res["sub_results"] = subs
        if a.cpu_seconds > 0:
            res["cpu_baseline"] = cpu_baseline_decode(wl, kv_bytes, a.cpu_seconds)
        from paged_kv_cache_175_amd import pool
        cfg = pool.PagedKVConfig(cache_dtype="f8e4m3" if wl.cache == "e4m3" else "auto",
                                 window=wl.window)
        res["describe"] = pool.describe(cfg, 1, wl.kv_read_tokens())
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
