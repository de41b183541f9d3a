"""GPU parity of pair mode: one split per sequence, where the workgroup of
each shorter sequence of a ranked pair also reads the tail of the longer one
and the longer one's workgroup merges the two partials (at once if the
helper has published, else whoever counts in last).

The batches mix long, short and empty sequences, odd and even batch sizes
(a middle sequence has no partner), rings whose lengths differ, the identity
map and the fused append (the helper patches the longer sequence's new row
into the page it reads).  Each output matches the oracle, on three calls in
a row on one workspace (the counters are back at zero after each).  The
waves of a workgroup claim pages as they go, so the summation order, and
the last bits, may differ from call to call.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import paritylib as P
from paged_kv_cache_175_amd import ops, pool
from paged_kv_cache_175_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = {
    # Long, short and one-token sequences (test_pair_decode empties one);
    # G = 4, D = 128.
    "mix_g4_d128": lambda: W.decode_workload("pair_mix", 91, B=6, Hq=32, Hkv=8, D=128,
                                             act="bf16", ctx=[4000, 1100, 2500, 1, 1, 3100]),
    # Odd batch: the middle sequence has no partner.
    "odd_f16_g8_d64": lambda: W.decode_workload("pair_odd", 92, B=9, Hq=16, Hkv=2, D=64,
                                                act="f16", ctx_range=(1, 5000)),
    "g2_d96": lambda: W.decode_workload("pair_d96", 93, B=12, Hq=8, Hkv=4, D=96, act="bf16",
                                        ctx_range=(300, 6000)),
    "mha_d64": lambda: W.decode_workload("pair_mha", 94, B=16, Hq=4, Hkv=4, D=64, act="bf16",
                                         ctx_range=(900, 3000)),
    # A ring of 1024 rows with positions below and above the window: the
    # lengths it reads differ.
    "ring_g4_d128": lambda: W.decode_workload("pair_ring", 95, B=7, Hq=32, Hkv=8, D=128,
                                              act="bf16", window=1024, pos_range=(50, 3000)),
    # One very long sequence among short ones, and two sequences.
    "one_long": lambda: W.decode_workload("pair_one_long", 96, B=5, Hq=8, Hkv=1, D=128,
                                          act="bf16", ctx=[8000, 40, 40, 40, 2000]),
    "two_seqs": lambda: W.decode_workload("pair_two", 97, B=2, Hq=8, Hkv=2, D=128, act="bf16",
                                          ctx=[6000, 1030]),
    # The largest batch pair mode takes.
    "b64": lambda: W.decode_workload("pair_b64", 98, B=64, Hq=8, Hkv=2, D=128, act="bf16",
                                     ctx_range=(0, 4096)),
}


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _oracle(wl):
    okc, ovc = P.oracle_decode_setup(wl)
    return P.oracle_decode(wl, okc, ovc)


def _pages(wl):
    L = np.minimum(wl.context_lens, wl.window) if wl.window else wl.context_lens
    return [int(-(-int(x) // 32)) for x in L]


@pytest.mark.parametrize("name", list(CASES))
def test_pair_decode(name):
    wl = CASES[name]()
    if name == "mix_g4_d128":
        wl.context_lens[4] = 0          # an empty sequence: zeros, and it still helps
    L = int(wl.context_lens.max())
    P.say(f"[pairs] {name} B={wl.B} pages={_pages(wl)}")
    assert ops.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, L, wl.window, 0,
                                      ops._lib.PA_BF16) > 0, "pair mode expected"
    kc, vc = P.hip_decode_setup(wl)
    q = P._act_tensor(wl.query, wl.act)
    ws = ops.alloc_workspace(ops.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, L,
                                                        wl.window, 0), q.device)
    outs = [ops.decode(q, kc, vc, _t(wl.block_tables), _t(wl.context_lens), L, wl.scale,
                       window=wl.window, workspace=ws).clone() for _ in range(3)]
    torch.cuda.synchronize()
    ref = _oracle(wl)
    errs = [P.max_abs(P.out_f64(o), ref) for o in outs]
    P.say(f"    max-abs error of the three calls {[f'{e:.3e}' for e in errs]}")
    assert max(errs) <= P.TOL[wl.act]
    # Every counter is back at zero.
    assert int(ws[:4 * max(wl.B * wl.Hkv, ops.MIN_COUNTERS)].count_nonzero()) == 0


@pytest.mark.parametrize("name", ["mix_g4_d128", "ring_g4_d128", "one_long", "b64"])
def test_pair_decode_append(name):
    wl = CASES[name]()
    P.say(f"[pairs append] {name} B={wl.B} pages={_pages(wl)}")
    kc, vc = P.hip_decode_append_setup(wl)
    out = P.hip_decode_append(wl, kc, vc)
    torch.cuda.synchronize()
    okc, ovc = P.oracle_decode_setup(wl)
    # The appended rows land exactly where the writer puts them.
    assert np.array_equal(P.pool_bits(kc), okc), "key pool differs"
    assert np.array_equal(P.pool_bits(vc), ovc), "value pool differs"
    err = P.max_abs(P.out_f64(out), P.oracle_decode(wl, okc, ovc))
    P.say(f"    max-abs error {err:.3e}")
    assert err <= P.TOL[wl.act]


@pytest.mark.parametrize("name", ["mix_g4_d128", "odd_f16_g8_d64"])
def test_pair_identity_map(name):
    wl = CASES[name]()
    B, M = wl.block_tables.shape
    wl = dataclasses.replace(wl, block_tables=pool.identity_table(B, M), num_blocks=B * M)
    P.say(f"[pairs identity] {name}")
    kc, vc = P.hip_decode_setup(wl)
    q = P._act_tensor(wl.query, wl.act)
    L = int(wl.context_lens.max())
    a = ops.decode(q, kc, vc, ops.IdentityMap(M), _t(wl.context_lens), L, wl.scale)
    b = ops.decode(q, kc, vc, _t(wl.block_tables), _t(wl.context_lens), L, wl.scale)
    torch.cuda.synchronize()
    P.same_output(a, b, P.TOL[wl.act], "identity map vs table")
    err = P.max_abs(P.out_f64(a), _oracle(wl))
    assert err <= P.TOL[wl.act]
