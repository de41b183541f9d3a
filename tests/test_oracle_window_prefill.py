"""Pins for the oracle's sliding-window chunked prefill into a ring (CPU).

The ring is filled position by position before the chunk (overwriting, as a
W-row ring does: "Rolling buffer cache", opening post); the chunk's own K/V
are passed separately.  Pinned against torch's fp64
``scaled_dot_product_attention`` over the *whole* history with an explicit
window mask ``i - W < pos <= i`` -- a computation that never sees the ring --
and against the ring decode of the token after the chunk once the chunk's
last W tokens are written into the ring.  Quantised rings (E4M3, INT8): a
one-token chunk equals the ring decode of that token once written, for
tokens that survive quantisation unchanged, and the ring's scales change the
result.
"""

import numpy as np
import pytest
import torch

from oracle import attention, cache, e4m3, int8
from paged_kv_cache_175_amd.workloads import to_act_bits


def _bits(rng, shape, act="bf16"):
    return to_act_bits(rng.standard_normal(shape).astype(np.float32), act)


def _setup(rng, W, BS, hist, C, Hq, Hkv, D, act="bf16"):
    """One sequence: positions 0..hist+C-1; the first `hist` are in the ring."""
    nblk = W // BS
    NB = nblk + 2
    order = rng.permutation(NB)
    bt = order[:nblk].astype(np.int32)[None, :]
    kc, vc = cache.empty_pools(NB, Hkv, BS, D, act, 0x7FC0)
    k_all = _bits(rng, (hist + C, Hkv, D), act)
    v_all = _bits(rng, (hist + C, Hkv, D), act)
    for pos in range(hist):
        slot = cache.slot_of(bt[0], pos % W, BS)
        cache.reshape_and_cache(k_all[pos:pos + 1], v_all[pos:pos + 1], kc, vc,
                                np.array([slot]), act, act)
    q = _bits(rng, (C, Hq, D), act)
    return kc, vc, bt, k_all, v_all, q


@pytest.mark.parametrize("W,BS,hist,C", [(16, 4, 40, 7), (16, 4, 5, 9), (8, 4, 30, 20),
                                         (12, 4, 0, 13), (16, 4, 16, 1)])
def test_window_prefill_equals_dense_masked(W, BS, hist, C):
    rng = np.random.default_rng(W * 1000 + hist * 10 + C)
    act, Hq, Hkv, D = "bf16", 4, 2, 8
    kc, vc, bt, k_all, v_all, q = _setup(rng, W, BS, hist, C, Hq, Hkv, D, act)
    ctx = hist + C
    out = attention.prefill_chunk_window(q, act, k_all[hist:], v_all[hist:], np.array([0, C]),
                                         kc, vc, act, bt, np.array([ctx]), 0.3, W)
    # Dense: every position's K/V, window mask for the chunk's queries.
    G = Hq // Hkv
    kd = np.repeat(cache.bits_to_f64(k_all, act).transpose(1, 0, 2), G, axis=0)
    vd = np.repeat(cache.bits_to_f64(v_all, act).transpose(1, 0, 2), G, axis=0)
    mask = np.full((C, ctx), -np.inf)
    for j in range(C):
        i = hist + j
        mask[j, max(0, i - W + 1):i + 1] = 0.0
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(cache.bits_to_f64(q, act).transpose(1, 0, 2))[None],
        torch.from_numpy(kd)[None], torch.from_numpy(vd)[None],
        attn_mask=torch.from_numpy(mask)[None, None], scale=0.3)[0].numpy()
    np.testing.assert_allclose(out, ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_ring_after_chunk_serves_the_next_decode():
    """Write the chunk's last W tokens into the ring, then the ring decode of
    the next token equals dense attention over its window."""
    rng = np.random.default_rng(77)
    act, W, BS, hist, C, Hq, Hkv, D = "bf16", 16, 4, 23, 21, 2, 1, 8
    kc, vc, bt, k_all, v_all, _ = _setup(rng, W, BS, hist, C + 1, Hq, Hkv, D, act)
    for pos in range(hist + max(0, C + 1 - W), hist + C + 1):   # chunk + next token
        slot = cache.slot_of(bt[0], pos % W, BS)
        cache.reshape_and_cache(k_all[pos:pos + 1], v_all[pos:pos + 1], kc, vc,
                                np.array([slot]), act, act)
    q = _bits(rng, (1, Hq, D), act)
    ctx = hist + C + 1
    out = attention.decode(q, act, kc, vc, act, bt, np.array([ctx]), 0.5, window=W)
    k = cache.bits_to_f64(k_all[ctx - W:ctx], act)
    v = cache.bits_to_f64(v_all[ctx - W:ctx], act)
    for h in range(Hq):
        ref = attention.softmax_attend(cache.bits_to_f64(q[0, h], act), k[:, 0], v[:, 0], 0.5)
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=1e-12)


def _exact_token(rng, fmt, Hkv, D, act, scale_pow):
    """K or V activations of one token that the cache stores without loss:
    E4M3 codes times a power-of-two scale, or INT8 codes (one of +-127 per
    row) times a power-of-two scale -- so quantising them gives the same
    values back."""
    s = np.float32(2.0 ** scale_pow)
    if fmt == "e4m3":
        codes = rng.integers(0, 0x7F, size=(1, Hkv, D))            # finite magnitudes
        codes = codes | (rng.integers(0, 2, (1, Hkv, D)) << 7)      # either sign
        vals = e4m3.decode(codes.astype(np.uint8), 1.0) * s
    else:
        codes = rng.integers(-126, 127, size=(1, Hkv, D)).astype(np.float64)
        codes[..., 0] = 127.0 * rng.choice([-1.0, 1.0], size=(1, Hkv))
        vals = codes * s
    return to_act_bits(vals.astype(np.float32), act), s


@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_quantised_ring_one_token_chunk_equals_ring_decode(fmt):
    """A one-token chunk over an E4M3 or INT8 ring equals the ring decode of
    that token once it is written, when the token's K/V survive quantisation
    unchanged: the chunk reads the ring's codes times their scales exactly as
    the decode does, and its own row from the activations."""
    rng = np.random.default_rng(5 if fmt == "e4m3" else 6)
    act, W, BS, hist, Hq, Hkv, D = "bf16", 16, 4, 37, 4, 2, 8
    nblk = W // BS
    NB = nblk + 2
    bt = rng.permutation(NB)[:nblk].astype(np.int32)[None, :]
    fill = 0x7F
    kc, vc = cache.empty_pools(NB, Hkv, BS, D, fmt, fill)
    if fmt == "e4m3":
        ksc, vsc = 0.25, 0.125
    else:
        ksc, vsc = cache.empty_scale_pools(NB, Hkv, BS, np.float32(np.nan))
    k_all = _bits(rng, (hist, Hkv, D), act)
    v_all = _bits(rng, (hist, Hkv, D), act)
    for pos in range(hist):
        slot = cache.slot_of(bt[0], pos % W, BS)
        cache.reshape_and_cache(k_all[pos:pos + 1], v_all[pos:pos + 1], kc, vc,
                                np.array([slot]), act, fmt, ksc, vsc)
    kn, _ = _exact_token(rng, fmt, Hkv, D, act, -2)
    vn, _ = _exact_token(rng, fmt, Hkv, D, act, -3)
    q = _bits(rng, (1, Hq, D), act)
    ctx = hist + 1
    out = attention.prefill_chunk_window(q, act, kn, vn, np.array([0, 1]), kc, vc, fmt, bt,
                                         np.array([ctx]), 0.4, W, k_scale=ksc, v_scale=vsc)
    slot = cache.slot_of(bt[0], hist % W, BS)
    cache.reshape_and_cache(kn, vn, kc, vc, np.array([slot]), act, fmt, ksc, vsc)
    # The token went into the cache unchanged.
    kr, vr = cache.get_row(kc, vc, slot // BS, slot % BS)
    if fmt == "e4m3":
        got_k = cache.bits_to_f64(kr, fmt) * 0.25
    else:
        got_k = int8.decode(kr, ksc[slot // BS, :, slot % BS])
    np.testing.assert_array_equal(got_k, cache.bits_to_f64(kn[0], act))
    ref = attention.decode(q, act, kc, vc, fmt, bt, np.array([ctx]), 0.4, ksc, vsc, window=W)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_quantised_ring_scales_matter():
    """The same E4M3 ring read with the wrong scale gives a different answer
    (the scale is applied to ring rows, not dropped)."""
    rng = np.random.default_rng(8)
    act, W, BS, hist, C, Hq, Hkv, D = "bf16", 8, 4, 20, 3, 2, 1, 8
    bt = np.arange(W // BS, dtype=np.int32)[None, :]
    kc, vc = cache.empty_pools(W // BS, Hkv, BS, D, "e4m3", 0x7F)
    k_all = _bits(rng, (hist + C, Hkv, D), act)
    v_all = _bits(rng, (hist + C, Hkv, D), act)
    for pos in range(hist):
        slot = cache.slot_of(bt[0], pos % W, BS)
        cache.reshape_and_cache(k_all[pos:pos + 1], v_all[pos:pos + 1], kc, vc,
                                np.array([slot]), act, "e4m3", 0.05, 0.05)
    q = _bits(rng, (C, Hq, D), act)
    args = (q, act, k_all[hist:], v_all[hist:], np.array([0, C]), kc, vc, "e4m3", bt,
            np.array([hist + C]), 0.4, W)
    a = attention.prefill_chunk_window(*args, k_scale=0.05, v_scale=0.05)
    b = attention.prefill_chunk_window(*args, k_scale=0.1, v_scale=0.05)
    c = attention.prefill_chunk_window(*args, k_scale=0.05, v_scale=0.1)
    assert np.max(np.abs(a - b)) > 1e-3 and np.max(np.abs(a - c)) > 1e-3
