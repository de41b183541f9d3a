"""pa_decode_noalloc, the decode entry point that allocates nothing (its
split scratch is a fixed array in the library's own device memory), against
pa_decode with a caller workspace, both through the C ABI.

Two calls in a row on one GPU, the second with a smaller input, then the
first again: each output matches pa_decode's on the same inputs and the
oracle within the output tolerance.  A 16-bit cache (split plan), an
E4M3 cache (balanced ranges) and an E4M3 batch in pair mode all use the
scratch.  The two entry points run
the same kernels with the same plan, but the waves of a workgroup claim
pages as they go, so the summation order, and the last bits, may differ
from one launch to the next.
"""

import pytest
import torch

import paritylib as P
from paged_kv_cache_175_amd import _lib, ops
from paged_kv_cache_175_amd import workloads as W

pytestmark = pytest.mark.gpu


def _noalloc(wl, kc, vc):
    q = P._act_tensor(wl.query, wl.act)
    bt = torch.from_numpy(wl.block_tables).cuda()
    cl = torch.from_numpy(wl.context_lens).cuda()
    out = torch.full_like(q, float("nan"))
    cache = ops._cache_code(kc, q.dtype)
    need = ops.decode_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, int(wl.context_lens.max()),
                                      wl.window, 0, cache)
    assert 0 < need <= _lib.PA_DECODE_SCRATCH_BYTES, "the case must use the scratch"
    _lib.check(_lib.load().pa_decode_noalloc(
        out.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(), bt.data_ptr(),
        cl.data_ptr(), wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, bt.shape[1],
        int(wl.context_lens.max()), wl.scale, ops._act_code(q), cache, wl.k_scale,
        wl.v_scale, wl.window, 0, torch.cuda.current_stream().cuda_stream))
    return out


@pytest.mark.parametrize("case", ["bf16", "e4m3", "e4m3_pairs"])
def test_noalloc_matches_pa_decode_twice(case):
    cache = case.split("_")[0]
    if case.endswith("pairs"):
        # 40 sequences x 8 KV heads from 1024 tokens: pair mode (one split per
        # sequence, short sequences help long ones through the scratch).
        big = W.decode_workload(f"noalloc_big_{case}", 43, B=40, Hq=32, Hkv=8, D=128,
                                act="bf16", cache=cache, ctx_range=(1024, 4000))
    else:
        big = W.decode_workload(f"noalloc_big_{case}", 41, B=6, Hq=32, Hkv=8, D=128,
                                act="bf16", cache=cache, ctx_range=(3000, 6000))
    small = W.decode_workload(f"noalloc_small_{cache}", 42, B=3, Hq=8, Hkv=2, D=64, act="bf16",
                              cache=cache, ctx_range=(1100, 2500))
    pools, refs = [], []
    for wl in (big, small):
        P.say(f"[noalloc] {wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} "
              f"ctx {wl.context_lens.min()}..{wl.context_lens.max()}")
        kc, vc = P.hip_decode_setup(wl)
        pools.append((kc, vc))
        refs.append(P.hip_decode(wl, kc, vc))          # pa_decode, caller workspace
    torch.cuda.synchronize()
    outs = [_noalloc(big, *pools[0]), _noalloc(small, *pools[1]), _noalloc(big, *pools[0])]
    torch.cuda.synchronize()
    tol = P.TOL[cache]
    for wl, ref, out in zip((big, small, big), refs + refs[:1], outs):
        diff = P.max_abs(P.out_f64(out), P.out_f64(ref))
        okc, ovc = P.oracle_decode_setup(wl)
        err = P.max_abs(P.out_f64(out), P.oracle_decode(wl, okc, ovc))
        P.say(f"[noalloc] {wl.name}: max-abs difference to pa_decode {diff:.2e}, "
              f"to the oracle {err:.2e}")
        assert diff <= tol, (wl.name, diff)
        assert err <= tol, (wl.name, err)
