"""Python binding of the paged KV-cache ops (thin marshalling over the C ABI).

Tensors are torch tensors on the GPU; torch provides device memory and the
current stream, nothing else.  Every op runs in the HIP kernels of
``libpagedkv.so``; there is no fallback path.

Cache dtypes follow the page "PagedAttention in mistral.rs", section "KV
Cache Quantization": ``"auto"`` stores the activation dtype, ``"f8e4m3"``
stores E4M3 codes (held in ``torch.uint8`` tensors) with per-tensor fp32
scales for K and V.  ``"i8"`` ("libmir-metal 0.2.0, src/native/trace/kv.rs",
fn build: packed INT8 pages with per-token/head FP32 scales) stores int8
codes in ``torch.int8`` pools plus fp32 scale pools ``[NB, Hkv, BS]``
(:func:`alloc_scale_pools`), passed as ``key_scales`` / ``value_scales``.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib, pool
from ._lib import PagedKVError  # noqa: F401  (re-export)

_ACT = {torch.float16: _lib.PA_F16, torch.bfloat16: _lib.PA_BF16}


def _act_code(t: torch.Tensor) -> int:
    try:
        return _ACT[t.dtype]
    except KeyError:
        raise TypeError(f"activation dtype must be float16 or bfloat16, got {t.dtype}") from None


def _cache_code(cache: torch.Tensor, act: torch.dtype) -> int:
    if cache.dtype == torch.uint8 or cache.dtype == getattr(torch, "float8_e4m3fn", None):
        return _lib.PA_F8E4M3
    if cache.dtype == torch.int8:
        return _lib.PA_I8
    if cache.dtype != act:
        raise TypeError(f"cache dtype {cache.dtype} must equal the activation dtype {act} "
                        "or be uint8 (E4M3 codes)")
    return _ACT[act]


def _dev(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _i32(*ts: torch.Tensor) -> None:
    for t in ts:
        if t.dtype != torch.int32:
            raise TypeError(f"index tensors must be int32, got {t.dtype}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class IdentityMap:
    """Stands in for ``block_tables`` when every sequence's blocks are the
    identity map: logical block j of sequence b is physical block
    ``b * max_blocks_per_seq + j`` (a dense ``[B][MBPS]`` pool).  The
    kernels then read no table (the C ABI's NULL ``block_tables``)."""

    def __init__(self, max_blocks_per_seq: int):
        if max_blocks_per_seq < 1:
            raise ValueError("max_blocks_per_seq must be positive")
        self.max_blocks_per_seq = int(max_blocks_per_seq)


def _table(block_tables, B: int):
    """(device pointer or 0, MBPS) of a ``[B, MBPS]`` int32 table or an
    :class:`IdentityMap`."""
    if isinstance(block_tables, IdentityMap):
        return 0, block_tables.max_blocks_per_seq
    _dev(block_tables)
    _i32(block_tables)
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B, MBPS]")
    return block_tables.data_ptr(), block_tables.shape[1]


def cache_dtype_name(cache: torch.Tensor) -> str:
    if cache.dtype == torch.uint8:
        return "f8e4m3"
    return "i8" if cache.dtype == torch.int8 else "auto"


def pool_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 32):
    """Shapes of the key and value pools.

    Key pages are ``[head_dim/8][block_size][8]`` and value pages
    ``[block_size/8][head_dim][8]`` (the layout of include/pa.h).
    """
    if head_dim % 8 or block_size % 8:
        raise ValueError("head_dim and block_size must be multiples of 8")
    return ((num_blocks, num_kv_heads, head_dim // 8, block_size, 8),
            (num_blocks, num_kv_heads, block_size // 8, head_dim, 8))


def _free_bytes(device) -> Optional[int]:
    device = torch.device(device)
    if device.type != "cuda":
        return None
    return torch.cuda.mem_get_info(device)[0]


def alloc_pools(num_blocks: int, num_kv_heads: int, head_dim: int, act_dtype: torch.dtype,
                cache_dtype: str = "auto", device="cuda", block_size: int = 32):
    """Allocate (uninitialised) key and value pools up front.  Raises
    :class:`pool.PoolTooLarge` before allocating when they exceed the
    device's free memory."""
    ks, vs = pool_shapes(num_blocks, num_kv_heads, head_dim, block_size)
    dt = {"f8e4m3": torch.uint8, "i8": torch.int8}.get(cache_dtype, act_dtype)
    elem = torch.empty((), dtype=dt).element_size()
    need = 2 * num_blocks * num_kv_heads * head_dim * block_size * elem
    pool.check_pool_fits(need, _free_bytes(device))
    return (torch.empty(ks, dtype=dt, device=device), torch.empty(vs, dtype=dt, device=device))


def alloc_model_pools(cfg: "pool.PagedKVConfig", num_kv_heads: int, head_dim: int,
                      act_dtype: torch.dtype, num_layers: int = 1, device="cuda"):
    """The pools of every layer of a model, sized by ``cfg`` (budget in MiB,
    fraction of free memory, or context size) and checked as a whole against
    the budget and the free memory before the first allocation.  Returns
    ``(num_blocks, [(key_cache, value_cache[, key_scales, value_scales]), ...])``."""
    act_bytes = torch.empty((), dtype=act_dtype).element_size()
    n = pool.plan_pool(cfg, num_kv_heads, head_dim, num_layers, act_bytes,
                       _free_bytes(device))
    layers = []
    for _ in range(num_layers):
        kc, vc = alloc_pools(n, num_kv_heads, head_dim, act_dtype, cfg.cache_dtype, device,
                             cfg.block_size)
        if cfg.cache_dtype == "i8":
            layers.append((kc, vc) + alloc_scale_pools(n, num_kv_heads, device, cfg.block_size))
        else:
            layers.append((kc, vc))
    return n, layers


def alloc_scale_pools(num_blocks: int, num_kv_heads: int, device="cuda", block_size: int = 32):
    """The fp32 per-row scale pools ``[NB, Hkv, BS]`` of an INT8 cache (K, V)."""
    shape = (num_blocks, num_kv_heads, block_size)
    return (torch.zeros(shape, dtype=torch.float32, device=device),
            torch.zeros(shape, dtype=torch.float32, device=device))


def _scales(cache_code, key_scales, value_scales, NB, Hkv, BS):
    """Scale-pool pointers of an INT8 cache (checked), else None."""
    if cache_code != _lib.PA_I8:
        if key_scales is not None or value_scales is not None:
            raise ValueError("scale pools belong to an int8 cache")
        return None
    if key_scales is None or value_scales is None:
        raise ValueError("an int8 cache needs key_scales and value_scales")
    _dev(key_scales, value_scales)
    for t in (key_scales, value_scales):
        if t.dtype != torch.float32 or tuple(t.shape) != (NB, Hkv, BS):
            raise ValueError(f"scale pools must be float32 [{NB}, {Hkv}, {BS}]")
    return key_scales.data_ptr(), value_scales.data_ptr()


def _pool_geometry(key_cache: torch.Tensor, value_cache: torch.Tensor):
    """(NB, Hkv, BS, D) of a pair of pools; raises on malformed shapes."""
    if key_cache.dim() != 5 or key_cache.shape[4] != 8 or value_cache.dim() != 5:
        raise ValueError("key_cache must be [NB, Hkv, D/8, BS, 8] and value_cache "
                         "[NB, Hkv, BS/8, D, 8]")
    NB, Hkv, D8, BS, _ = key_cache.shape
    if (BS % 8 or tuple(value_cache.shape) != (NB, Hkv, BS // 8, D8 * 8, 8)
            or value_cache.dtype != key_cache.dtype):
        raise ValueError("value_cache does not match key_cache")
    return NB, Hkv, BS, D8 * 8


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, slot_mapping: torch.Tensor,
                      k_scale: float = 1.0, v_scale: float = 1.0,
                      key_scales: Optional[torch.Tensor] = None,
                      value_scales: Optional[torch.Tensor] = None) -> None:
    """Write ``key``/``value`` ``[T, Hkv, D]`` into the pools at ``slot_mapping``.

    Pools as from :func:`alloc_pools`; a negative slot skips its token.  An
    int8 cache also writes each row's scale into ``key_scales`` /
    ``value_scales``.
    """
    _dev(key, value, key_cache, value_cache, slot_mapping)
    _i32(slot_mapping)
    if key.shape != value.shape or key.dim() != 3:
        raise ValueError("key and value must both be [T, Hkv, D]")
    T, Hkv, D = key.shape
    NB, Hc, BS, Dc = _pool_geometry(key_cache, value_cache)
    if (Hc, Dc) != (Hkv, D) or slot_mapping.numel() != T:
        raise ValueError("shape mismatch between tokens, caches and slot_mapping")
    act = _act_code(key)
    cache = _cache_code(key_cache, key.dtype)
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS)
    lib = _lib.load()
    if sc is not None:
        _lib.check(lib.pa_reshape_and_cache_i8(
            key.data_ptr(), value.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            *sc, slot_mapping.data_ptr(), T, Hkv, D, BS, NB, act, _stream()))
        return
    _lib.check(lib.pa_reshape_and_cache(
        key.data_ptr(), value.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        slot_mapping.data_ptr(), T, Hkv, D, BS, NB, act, cache, float(k_scale), float(v_scale),
        _stream()))


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_mapping: torch.Tensor,
                key_scales: Optional[torch.Tensor] = None,
                value_scales: Optional[torch.Tensor] = None) -> None:
    """Copy whole blocks ``block_mapping`` ``[N, 2]`` (src, dst) in the pools
    (and an int8 cache's scale pools): the copies a sequence's
    copy-on-write queues (:meth:`pool.SequenceBlocks.take_copies`)."""
    _dev(key_cache, value_cache, block_mapping)
    _i32(block_mapping)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [N, 2]")
    NB, Hkv, BS, D = _pool_geometry(key_cache, value_cache)
    cache = _cache_code(key_cache, torch.bfloat16 if key_cache.dtype != torch.float16
                        else torch.float16)
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS) or (0, 0)
    _lib.check(_lib.load().pa_copy_blocks(
        key_cache.data_ptr(), value_cache.data_ptr(), sc[0], sc[1], block_mapping.data_ptr(),
        block_mapping.shape[0], Hkv, D, BS, NB, cache, _stream()))


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, max_context_len: int,
                           window: int = 0, partition_tokens: int = 0,
                           cache_dtype: Optional[int] = None) -> int:
    """Workspace bytes of a decode call; with ``cache_dtype`` (a PA_* code)
    exactly that format's need, else the largest over the formats."""
    lib = _lib.load()
    if cache_dtype is None:
        n = lib.pa_decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, window,
                                          partition_tokens)
    else:
        n = lib.pa_decode_workspace_bytes_for(B, Hq, Hkv, D, max_context_len, window,
                                              partition_tokens, int(cache_dtype))
    if n == (1 << 64) - 1:
        raise PagedKVError(_lib.PA_ERR_INVALID, "invalid workspace query")
    return int(n)


# The decode workspace begins with its split arrival counters: 4 bytes per
# (sequence, KV head), at least MIN_COUNTERS of them (include/pa.h).  They
# must be zero when a call starts; a call leaves its own counters at zero and
# writes its partials just past its counter region.  So once zeroed, the
# counters stay valid for every later call whose B * Hkv does not exceed that
# of the last call that wrote partials (or MIN_COUNTERS); a larger one finds
# partials where its counters lie and has them zeroed first.  A workspace
# tensor records how many leading counters are known to be zero.
MIN_COUNTERS = 16384
_CLEAN = "_pa_clean_counters"


def alloc_workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """Decode workspace, zero-filled: reusable across calls of any shape
    through :func:`decode` / :func:`prepare_decode`, which zero its counters
    again when a call has more (sequence, KV head) pairs than the workspace
    is known to have clean."""
    if nbytes == 0:
        return None
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    setattr(ws, _CLEAN, nbytes // 4)
    return ws


def _check_workspace(workspace: torch.Tensor, device) -> None:
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if workspace.device != device:
        raise ValueError(f"workspace is on {workspace.device}, the query on {device}")


def _ready_counters(workspace: Optional[torch.Tensor], need: int, pairs: int) -> None:
    """Zero the workspace's counters for a call over ``pairs`` (sequence, KV
    head) pairs if they may hold partials of an earlier call, then record
    what the call leaves clean."""
    if workspace is None or need == 0:
        return
    clean = getattr(workspace, _CLEAN, MIN_COUNTERS)
    if pairs > clean:
        workspace[:4 * pairs].zero_()
    # The call writes partials from its counter region's end on.
    setattr(workspace, _CLEAN, max(pairs, MIN_COUNTERS))


def _check_out(out: torch.Tensor, like: torch.Tensor) -> None:
    if out.shape != like.shape or out.dtype != like.dtype or out.device != like.device:
        raise ValueError(f"out must be {tuple(like.shape)} {like.dtype} on {like.device}")
    _dev(out)


def decode(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
           softmax_scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
           window: int = 0, partition_tokens: int = 0, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, new_key: Optional[torch.Tensor] = None,
           new_value: Optional[torch.Tensor] = None,
           key_scales: Optional[torch.Tensor] = None,
           value_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged decode attention; returns ``out`` ``[B, Hq, D]``.

    ``workspace`` (uint8, >= :func:`decode_workspace_bytes`) is allocated here
    when not given.  With ``new_key`` / ``new_value`` (``[B, Hkv, D]``) the
    decoded token is first stored into its cache row in the same launch
    (``pa_decode_append``).  An int8 cache reads its scale pools
    ``key_scales`` / ``value_scales`` (``pa_decode_i8``; with the new token,
    ``pa_decode_append_i8`` writes its codes and row scales).
    """
    _dev(query, key_cache, value_cache, context_lens)
    _i32(context_lens)
    B, Hq, D = query.shape
    NB, Hkv, BS, Dc = _pool_geometry(key_cache, value_cache)
    if Dc != D:
        raise ValueError("cache shapes do not match the query")
    if context_lens.numel() != B:
        raise ValueError("context_lens must be [B]")
    bt_ptr, MBPS = _table(block_tables, B)
    act = _act_code(query)
    cache = _cache_code(key_cache, query.dtype)
    if out is None:
        out = torch.empty_like(query)
    _check_out(out, query)
    need = decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, window, partition_tokens,
                                  cache)
    if workspace is None:
        workspace = alloc_workspace(need, query.device)
    else:
        _check_workspace(workspace, query.device)
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel()
    if ws_bytes < need:
        raise PagedKVError(_lib.PA_ERR_WORKSPACE, f"workspace needs {need} bytes (got {ws_bytes})")
    _ready_counters(workspace, need, B * Hkv)
    lib = _lib.load()
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS)
    if sc is not None:
        tail_i8 = (bt_ptr, context_lens.data_ptr(), B, Hq, Hkv, D, BS, MBPS,
                   int(max_context_len), float(softmax_scale), act, int(window),
                   int(partition_tokens), ws_ptr, ws_bytes, _stream())
        if new_key is None:
            _lib.check(lib.pa_decode_i8(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(),
                                        value_cache.data_ptr(), *sc, *tail_i8))
        else:
            _check_new_token(new_key, new_value, query, Hkv, D)
            _lib.check(lib.pa_decode_append_i8(
                out.data_ptr(), query.data_ptr(), new_key.data_ptr(), new_value.data_ptr(),
                key_cache.data_ptr(), value_cache.data_ptr(), *sc, *tail_i8))
        return out
    tail = (bt_ptr, context_lens.data_ptr(), B, Hq, Hkv, D, BS, MBPS,
            int(max_context_len), float(softmax_scale), act, cache, float(k_scale),
            float(v_scale), int(window), int(partition_tokens), ws_ptr, ws_bytes, _stream())
    if new_key is None:
        _lib.check(lib.pa_decode(out.data_ptr(), query.data_ptr(), key_cache.data_ptr(),
                                 value_cache.data_ptr(), *tail))
    else:
        _check_new_token(new_key, new_value, query, Hkv, D)
        _lib.check(lib.pa_decode_append(out.data_ptr(), query.data_ptr(), new_key.data_ptr(),
                                        new_value.data_ptr(), key_cache.data_ptr(),
                                        value_cache.data_ptr(), *tail))
    return out


def _check_new_token(new_key, new_value, query, Hkv, D):
    _dev(new_key, new_value)
    B = query.shape[0]
    if new_value is None or new_key.shape != (B, Hkv, D) or new_value.shape != (B, Hkv, D):
        raise ValueError("new_key / new_value must both be [B, Hkv, D]")
    if new_key.dtype != query.dtype or new_value.dtype != query.dtype:
        raise TypeError("new_key / new_value must have the activation dtype")


def prefill_chunk(query: torch.Tensor, cu_q_lens: torch.Tensor, key_cache: torch.Tensor,
                  value_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, max_chunk_len: int, softmax_scale: float,
                  k_scale: float = 1.0, v_scale: float = 1.0,
                  out: Optional[torch.Tensor] = None,
                  key_scales: Optional[torch.Tensor] = None,
                  value_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal chunked prefill over the paged cache; returns ``out`` ``[total_q, Hq, D]``.

    ``softmax_scale`` must be finite and > 0 (the library rejects others).
    An int8 cache reads its scale pools (``pa_prefill_chunk_i8``)."""
    _dev(query, cu_q_lens, key_cache, value_cache, context_lens)
    _i32(cu_q_lens, context_lens)
    total_q, Hq, D = query.shape
    NB, Hkv, BS, Dc = _pool_geometry(key_cache, value_cache)
    B = context_lens.numel()
    if Dc != D:
        raise ValueError("cache shapes do not match the query")
    if cu_q_lens.numel() != B + 1:
        raise ValueError("cu_q_lens must be [B+1]")
    bt_ptr, MBPS = _table(block_tables, B)
    act = _act_code(query)
    cache = _cache_code(key_cache, query.dtype)
    if out is None:
        out = torch.empty_like(query)
    _check_out(out, query)
    lib = _lib.load()
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS)
    if sc is not None:
        _lib.check(lib.pa_prefill_chunk_i8(
            out.data_ptr(), query.data_ptr(), cu_q_lens.data_ptr(), key_cache.data_ptr(),
            value_cache.data_ptr(), *sc, bt_ptr, context_lens.data_ptr(), B,
            Hq, Hkv, D, BS, MBPS, int(max_chunk_len), float(softmax_scale), act, _stream()))
        return out
    _lib.check(lib.pa_prefill_chunk(
        out.data_ptr(), query.data_ptr(), cu_q_lens.data_ptr(), key_cache.data_ptr(),
        value_cache.data_ptr(), bt_ptr, context_lens.data_ptr(), B, Hq, Hkv,
        D, BS, MBPS, int(max_chunk_len), float(softmax_scale), act, cache, float(k_scale),
        float(v_scale), _stream()))
    return out


def prefill_chunk_window(query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                         cu_q_lens: torch.Tensor, key_cache: torch.Tensor,
                         value_cache: torch.Tensor, block_tables: torch.Tensor,
                         context_lens: torch.Tensor, max_chunk_len: int, softmax_scale: float,
                         window: int, out: Optional[torch.Tensor] = None,
                         k_scale: float = 1.0, v_scale: float = 1.0,
                         key_scales: Optional[torch.Tensor] = None,
                         value_scales: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunked prefill of a sliding-window layer over its ring
    (``pa_prefill_chunk_window``); ``key`` / ``value`` ``[total_q, Hkv, D]``
    are the chunk's own K/V, written into the ring only after this call.  An
    E4M3 ring (uint8) reads with ``k_scale`` / ``v_scale``, an INT8 ring
    with its scale pools (``pa_prefill_chunk_window_quant``).
    ``softmax_scale`` must be finite and > 0."""
    _dev(query, key, value, cu_q_lens, key_cache, value_cache, context_lens)
    _i32(cu_q_lens, context_lens)
    total_q, Hq, D = query.shape
    NB, Hkv, BS, Dc = _pool_geometry(key_cache, value_cache)
    B = context_lens.numel()
    if Dc != D:
        raise ValueError("cache shapes do not match the query")
    if key.shape != (total_q, Hkv, D) or value.shape != (total_q, Hkv, D):
        raise ValueError("key / value must both be [total_q, Hkv, D]")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise TypeError("key / value must have the activation dtype")
    if cu_q_lens.numel() != B + 1:
        raise ValueError("cu_q_lens must be [B+1]")
    bt_ptr, MBPS = _table(block_tables, B)
    act = _act_code(query)
    cache = _cache_code(key_cache, query.dtype)
    if out is None:
        out = torch.empty_like(query)
    _check_out(out, query)
    if cache == act:
        _lib.check(_lib.load().pa_prefill_chunk_window(
            out.data_ptr(), query.data_ptr(), key.data_ptr(), value.data_ptr(),
            cu_q_lens.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            bt_ptr, context_lens.data_ptr(), B, Hq, Hkv, D, BS,
            MBPS, int(max_chunk_len), float(softmax_scale), act, int(window),
            _stream()))
        return out
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS) or (0, 0)
    _lib.check(_lib.load().pa_prefill_chunk_window_quant(
        out.data_ptr(), query.data_ptr(), key.data_ptr(), value.data_ptr(),
        cu_q_lens.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), sc[0], sc[1],
        bt_ptr, context_lens.data_ptr(), B, Hq, Hkv, D, BS, MBPS, int(max_chunk_len),
        float(softmax_scale), act, cache, float(k_scale), float(v_scale), int(window),
        _stream()))
    return out


# ---------------------------------------------------------------------------
# Prepared calls: all marshalling done once, so that a tight loop (or a HIP
# graph capture) pays only the ctypes call.  The returned callables launch on
# the stream that was current when they were prepared.


def prepare_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping,
                              k_scale: float = 1.0, v_scale: float = 1.0,
                              key_scales=None, value_scales=None):
    _dev(key, value, key_cache, value_cache, slot_mapping)
    _i32(slot_mapping)
    T, Hkv, D = key.shape
    NB, _, BS, _ = _pool_geometry(key_cache, value_cache)
    lib = _lib.load()
    cache = _cache_code(key_cache, key.dtype)
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS)
    if sc is not None:
        args = (key.data_ptr(), value.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                *sc, slot_mapping.data_ptr(), T, Hkv, D, BS, NB, _act_code(key), _stream())
        fn = lib.pa_reshape_and_cache_i8
    else:
        args = (key.data_ptr(), value.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
                slot_mapping.data_ptr(), T, Hkv, D, BS, NB, _act_code(key), cache,
                float(k_scale), float(v_scale), _stream())
        fn = lib.pa_reshape_and_cache

    def call():
        _lib.check(fn(*args))
    return call


def prepare_decode(query, key_cache, value_cache, block_tables, context_lens,
                   max_context_len: int, softmax_scale: float, out, workspace=None,
                   k_scale: float = 1.0, v_scale: float = 1.0, window: int = 0,
                   partition_tokens: int = 0, new_key=None, new_value=None,
                   key_scales=None, value_scales=None):
    _dev(query, key_cache, value_cache, context_lens)
    _i32(context_lens)
    _check_out(out, query)
    B, Hq, D = query.shape
    NB, Hkv, BS, _ = _pool_geometry(key_cache, value_cache)
    bt_ptr, MBPS = _table(block_tables, B)
    need = decode_workspace_bytes(B, Hq, Hkv, D, max_context_len, window, partition_tokens,
                                  _cache_code(key_cache, query.dtype))
    if workspace is not None:
        _check_workspace(workspace, query.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    if ws_bytes < need:
        raise PagedKVError(_lib.PA_ERR_WORKSPACE, f"workspace needs {need} bytes")
    pairs = B * Hkv
    lib = _lib.load()
    cache = _cache_code(key_cache, query.dtype)
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS)
    tail = (bt_ptr, context_lens.data_ptr(), B, Hq, Hkv, D, BS, MBPS,
            int(max_context_len), float(softmax_scale), _act_code(query), cache,
            float(k_scale), float(v_scale), int(window), int(partition_tokens), ws_ptr,
            ws_bytes, _stream())
    if sc is not None:
        tail_i8 = (bt_ptr, context_lens.data_ptr(), B, Hq, Hkv, D, BS, MBPS,
                   int(max_context_len), float(softmax_scale), _act_code(query), int(window),
                   int(partition_tokens), ws_ptr, ws_bytes, _stream())
        if new_key is None:
            args = (out.data_ptr(), query.data_ptr(), key_cache.data_ptr(),
                    value_cache.data_ptr(), *sc) + tail_i8
            fn = lib.pa_decode_i8
        else:
            _check_new_token(new_key, new_value, query, Hkv, D)
            args = (out.data_ptr(), query.data_ptr(), new_key.data_ptr(), new_value.data_ptr(),
                    key_cache.data_ptr(), value_cache.data_ptr(), *sc) + tail_i8
            fn = lib.pa_decode_append_i8
    elif new_key is None:
        args = (out.data_ptr(), query.data_ptr(), key_cache.data_ptr(),
                value_cache.data_ptr()) + tail
        fn = lib.pa_decode
    else:
        _check_new_token(new_key, new_value, query, Hkv, D)
        args = (out.data_ptr(), query.data_ptr(), new_key.data_ptr(), new_value.data_ptr(),
                key_cache.data_ptr(), value_cache.data_ptr()) + tail
        fn = lib.pa_decode_append

    # The counter check is host-side bookkeeping: a zero fill is launched
    # only when another call's partials may lie where this call's counters do.
    _ready_counters(workspace, need, pairs)

    def call():
        _ready_counters(workspace, need, pairs)
        _lib.check(fn(*args))
    return call


def prepare_prefill_chunk(query, cu_q_lens, key_cache, value_cache, block_tables, context_lens,
                          max_chunk_len: int, softmax_scale: float, out,
                          k_scale: float = 1.0, v_scale: float = 1.0,
                          key_scales=None, value_scales=None):
    _dev(query, cu_q_lens, key_cache, value_cache, context_lens)
    _i32(cu_q_lens, context_lens)
    _check_out(out, query)
    total_q, Hq, D = query.shape
    NB, Hkv, BS, _ = _pool_geometry(key_cache, value_cache)
    B = context_lens.numel()
    bt_ptr, MBPS = _table(block_tables, B)
    lib = _lib.load()
    cache = _cache_code(key_cache, query.dtype)
    sc = _scales(cache, key_scales, value_scales, NB, Hkv, BS)
    if sc is not None:
        args = (out.data_ptr(), query.data_ptr(), cu_q_lens.data_ptr(), key_cache.data_ptr(),
                value_cache.data_ptr(), *sc, bt_ptr, context_lens.data_ptr(),
                B, Hq, Hkv, D, BS, MBPS, int(max_chunk_len), float(softmax_scale),
                _act_code(query), _stream())
        fn = lib.pa_prefill_chunk_i8
    else:
        args = (out.data_ptr(), query.data_ptr(), cu_q_lens.data_ptr(), key_cache.data_ptr(),
                value_cache.data_ptr(), bt_ptr, context_lens.data_ptr(), B, Hq,
                Hkv, D, BS, MBPS, int(max_chunk_len), float(softmax_scale), _act_code(query),
                cache, float(k_scale), float(v_scale), _stream())
        fn = lib.pa_prefill_chunk

    def call():
        _lib.check(fn(*args))
    return call
