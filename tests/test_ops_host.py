"""Host logic of the Python binding (no GPU): the decode workspace's counter
bookkeeping and the checks on ``out`` and ``workspace`` that run before any
library call."""

import pytest
import torch

from paged_kv_cache_175_amd import ops

MIN = ops.MIN_COUNTERS


def _clean(ws):
    return getattr(ws, ops._CLEAN)


def test_fresh_workspace_is_clean():
    ws = ops.alloc_workspace(1 << 20, "cpu")
    assert int(ws.abs().sum()) == 0 and _clean(ws) == (1 << 20) // 4
    assert ops.alloc_workspace(0, "cpu") is None


def test_counters_zeroed_only_where_partials_may_lie():
    n = 4 * (MIN + 4096)
    ws = ops.alloc_workspace(n, "cpu")
    # A call over few pairs leaves clean only its own counter region (the
    # minimum): its partials start right after it.
    ops._ready_counters(ws, 1, 100)
    assert _clean(ws) == MIN
    ws[4 * MIN:] = 0xAB                      # that call's partials
    # A call over more pairs finds partials where its counters lie: zeroed.
    ops._ready_counters(ws, 1, MIN + 1000)
    assert int(ws[:4 * (MIN + 1000)].abs().sum()) == 0
    assert bool((ws[4 * (MIN + 1000):] == 0xAB).all())      # nothing else touched
    assert _clean(ws) == MIN + 1000
    ws[4 * (MIN + 1000):] = 0xCD
    # Fewer pairs than are clean: no fill; the call's partials then start
    # after its smaller region.
    ops._ready_counters(ws, 1, MIN + 500)
    assert bool((ws[4 * (MIN + 1000):] == 0xCD).all())
    assert _clean(ws) == MIN + 500
    ws[4 * (MIN + 500):] = 0xEF
    ops._ready_counters(ws, 1, MIN + 1000)
    assert int(ws[:4 * (MIN + 1000)].abs().sum()) == 0
    # A call that needs no workspace changes nothing.
    ops._ready_counters(ws, 0, 10 * MIN)
    assert _clean(ws) == MIN + 1000


def test_unknown_workspace_assumes_the_minimum_region():
    ws = torch.full((4 * (MIN + 64),), 0x11, dtype=torch.uint8)
    ws[:4 * MIN] = 0                         # the caller zero-filled the counter region
    ops._ready_counters(ws, 1, MIN + 64)
    assert int(ws.abs().sum()) == 0


def test_out_and_workspace_checks():
    q = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be"):
        ops._check_out(torch.zeros(2, 8, 64, dtype=torch.float16), q)
    with pytest.raises(ValueError, match="out must be"):
        ops._check_out(torch.zeros(2, 8, 32, dtype=torch.bfloat16), q)
    with pytest.raises(ValueError, match="on the GPU"):
        ops._check_out(torch.zeros(2, 8, 64, dtype=torch.bfloat16), q)
    with pytest.raises(ValueError, match="uint8"):
        ops._check_workspace(torch.zeros(64, dtype=torch.float32), q.device)
    with pytest.raises(ValueError, match="uint8"):
        ops._check_workspace(torch.zeros(8, 8, dtype=torch.uint8), q.device)
    with pytest.raises(ValueError, match="contiguous"):
        ops._check_workspace(torch.zeros(128, dtype=torch.uint8)[::2], q.device)
    with pytest.raises(ValueError, match="workspace is on"):
        ops._check_workspace(torch.zeros(64, dtype=torch.uint8, device="meta"), q.device)
    ops._check_workspace(torch.zeros(64, dtype=torch.uint8), q.device)
