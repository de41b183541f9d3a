"""GPU parity of copy-on-write: the block copy kernel against the oracle's
block copy (bit for bit, every format), and a fork/append scenario run
through the HIP copy, writer and decode against the oracle doing the same
steps."""

import numpy as np
import pytest
import torch

import paritylib as P
from oracle import attention as o_attn
from oracle import cache as o_cache
from paged_kv_cache_175_amd import ops, pool
from paged_kv_cache_175_amd.workloads import to_act_bits

pytestmark = pytest.mark.gpu

DEV = "cuda"
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "e4m3": torch.uint8, "int8": torch.int8}


def _to_gpu(a, fmt):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if fmt in ("bf16", "f16"):
        t = t.view(torch.int16).view(TORCH_DT[fmt])
    return t.to(DEV)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "e4m3", "int8"])
def test_copy_blocks_bitwise(fmt):
    rng = np.random.default_rng(7)
    NB, Hkv, D = 12, 4, 96
    kc, vc = o_cache.empty_pools(NB, Hkv, 32, D, fmt)
    kc[...] = rng.integers(0, 1 << 14, kc.shape).astype(kc.dtype)
    vc[...] = rng.integers(0, 1 << 14, vc.shape).astype(vc.dtype)
    ks = vs = None
    if fmt == "int8":
        ks, vs = o_cache.empty_scale_pools(NB, Hkv, 32)
        ks[...] = rng.random(ks.shape)
        vs[...] = rng.random(vs.shape)
    mapping = np.array([[3, 7], [3, 9], [0, 11], [5, 1]], dtype=np.int32)
    gk, gv = _to_gpu(kc, fmt), _to_gpu(vc, fmt)
    gks = None if ks is None else torch.from_numpy(ks).to(DEV)
    gvs = None if vs is None else torch.from_numpy(vs).to(DEV)
    P.say(f"[copy_blocks] {fmt} pairs={mapping.tolist()}")
    ops.copy_blocks(gk, gv, torch.from_numpy(mapping).to(DEV), gks, gvs)
    torch.cuda.synchronize()
    o_cache.copy_blocks(kc, vc, mapping, ks, vs)
    assert np.array_equal(P.pool_bits(gk), kc.view(P.pool_bits(gk).dtype))
    assert np.array_equal(P.pool_bits(gv), vc.view(P.pool_bits(gv).dtype))
    if ks is not None:
        assert np.array_equal(gks.cpu().numpy(), ks) and np.array_equal(gvs.cpu().numpy(), vs)


def test_fork_append_decode_scenario():
    rng = np.random.default_rng(8)
    act, Hq, Hkv, D, BS, NB = "bf16", 8, 2, 64, 32, 48
    order = rng.permutation(NB)
    g_alloc = pool.BlockAllocator(NB, order=order)
    o_alloc = pool.BlockAllocator(NB, order=order)
    kshape, vshape = ops.pool_shapes(NB, Hkv, D, BS)
    gk = torch.full(kshape, 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    gv = torch.full(vshape, 0x7FC0, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    okc, ovc = o_cache.empty_pools(NB, Hkv, BS, D, act, 0x7FC0)
    gseqs, oseqs = [pool.SequenceBlocks(g_alloc, BS)], [pool.SequenceBlocks(o_alloc, BS)]
    copies_seen = 0
    for step in range(30):
        i = int(rng.integers(len(gseqs)))
        if rng.random() < 0.3 and len(gseqs) < 6 and gseqs[i].num_tokens:
            gseqs.append(gseqs[i].fork())
            oseqs.append(oseqs[i].fork())
            continue
        n = int(rng.integers(1, 50))
        gs, os_ = gseqs[i].append(n), oseqs[i].append(n)
        gc, oc = gseqs[i].take_copies(), oseqs[i].take_copies()
        assert gs == os_ and np.array_equal(gc, oc)
        copies_seen += len(gc)
        if len(gc):
            ops.copy_blocks(gk, gv, torch.from_numpy(gc).to(DEV))
            o_cache.copy_blocks(okc, ovc, oc)
        k = to_act_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32), act)
        v = to_act_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32), act)
        ops.reshape_and_cache(P._act_tensor(k, act), P._act_tensor(v, act), gk, gv,
                              torch.tensor(gs, dtype=torch.int32, device=DEV))
        o_cache.reshape_and_cache(k, v, okc, ovc, np.array(os_), act, act)
    torch.cuda.synchronize()
    P.say(f"[cow scenario] sequences={len(gseqs)} copies={copies_seen} "
          f"lens={[s.num_tokens for s in gseqs]}")
    assert copies_seen > 0
    assert np.array_equal(P.pool_bits(gk), okc) and np.array_equal(P.pool_bits(gv), ovc)
    live = [s for s in gseqs if s.num_tokens]
    bt = pool.block_table_array(live, pad=0)
    lens = np.array([s.num_tokens for s in live], dtype=np.int32)
    q = to_act_bits(rng.standard_normal((len(live), Hq, D)).astype(np.float32), act)
    out = ops.decode(P._act_tensor(q, act), gk, gv, torch.from_numpy(bt).to(DEV),
                     torch.from_numpy(lens).to(DEV), int(lens.max()), 0.125)
    ref = o_attn.decode(q, act, okc, ovc, act, bt, lens, 0.125)
    err = P.max_abs(P.out_f64(out), ref)
    P.say(f"    max-abs error {err:.3e}")
    assert err <= P.TOL[act]
