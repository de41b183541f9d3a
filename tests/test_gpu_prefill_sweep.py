"""Causal chunked prefill over a shared prefix against the oracle, over a
seeded sweep of shapes: prefixes of 0 to 12 blocks, chunks of 0 to 400
tokens (so the context ends at every row of a page and the page ranges have
odd and even lengths, which the 16-bit path stages in pairs), 1 to 4
sequences, 1 or 2 KV heads with 1, 2, 4 or 8 query heads each.  Every cache
format (the activation format, E4M3, INT8), head size (64, 96, 128) and
activation format (bf16, f16) comes up.

Checked, as in the fixed cases: the pools byte for byte against the
oracle's writer (INT8: the row scales too) and the output within the cache
format's tolerance.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paritylib as P
from paged_kv_cache_175_amd import workloads as W

pytestmark = pytest.mark.gpu

N_CASES = 36
CACHES = (None, "e4m3", "int8")   # None: the activation format
HEAD_DIMS = (64, 96, 128)
ACTS = ("bf16", "f16")


def _case(i: int) -> dict:
    """Case i: the format, head size and activation cycle so that every
    combination appears twice; the rest is drawn from a generator seeded
    by i."""
    rng = np.random.default_rng(7000 + i)
    B = int(rng.integers(1, 5))
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8]))
    chunks = [int(rng.integers(0, 401)) for _ in range(B)]
    if max(chunks) == 0:
        chunks[0] = 1
    return dict(cache=CACHES[i % 3], D=HEAD_DIMS[(i // 3) % 3], act=ACTS[(i // 9) % 2], B=B,
                Hkv=Hkv, Hq=G * Hkv, prefix_len=32 * int(rng.integers(0, 13)), chunks=chunks,
                seed=8000 + i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_prefill_sweep(i):
    c = _case(i)
    wl = W.prefill_workload(f"psweep_{i}", c["seed"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"],
                            D=c["D"], act=c["act"], prefix_len=c["prefix_len"],
                            chunks=c["chunks"], cache=c["cache"])
    P.say(f"[prefill sweep {i}] cache {c['cache'] or c['act']} D={c['D']} act={c['act']} "
          f"B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} prefix={c['prefix_len']} "
          f"chunks={c['chunks']}")
    if c["cache"] == "int8":
        pools = P.hip_prefill_setup_i8(wl)
        out = P.hip_prefill_i8(wl, pools)
        torch.cuda.synchronize()
        opools = P.oracle_prefill_setup_i8(wl)
        for got, ref, what in zip(pools, opools, ("key codes", "value codes", "key scales",
                                                 "value scales")):
            g = P.scale_bits(got) if got.dtype == torch.float32 else P.pool_bits(got)
            r = ref.view(np.int32) if ref.dtype == np.float32 else ref
            assert np.array_equal(g, r), what
        ref = P.oracle_prefill_i8(wl, opools)
        tol = P.TOL["int8"]
    else:
        kc, vc = P.hip_prefill_setup(wl)
        out = P.hip_prefill(wl, kc, vc)
        torch.cuda.synchronize()
        okc, ovc = P.oracle_prefill_setup(wl)
        assert np.array_equal(P.pool_bits(kc), okc), "key pool bytes differ"
        assert np.array_equal(P.pool_bits(vc), ovc), "value pool bytes differ"
        ref = P.oracle_prefill(wl, okc, ovc)
        tol = P.TOL[wl.cache]
    err = P.max_abs(P.out_f64(out), ref)
    P.say(f"    max-abs error {err:.3e} (tolerance {tol:.0e})")
    assert err <= tol
