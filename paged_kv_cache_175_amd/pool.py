"""Host-side block manager: pool sizing, block allocation, block tables and
slot mappings (full cache and rolling buffer), shared prefix blocks, models
mixing full and sliding-window layers.

What the pages fix ("PagedAttention in mistral.rs"):

* the pool has two inputs, a GPU memory budget in MB and a block size in
  tokens (default 32); the budget may also be a fraction of GPU memory or,
  in the Rust API, a context size in tokens;
* the pool is allocated up front, which is why an oversized budget shows up
  as an out-of-memory error;
* an F8E4M3 cache about halves the memory of an FP16 one;
* prefix caching reuses cached prefix KV across requests; the libmir-metal
  trace page ("libmir-metal 0.2.0, src/native/trace/kv.rs", fn build) names
  copy-on-write page maps for the shared pages.

Copy-on-write (a reading: the pages name it without rules): a sequence may
share another's blocks up to any position, a partially filled last block
included.  A block is shared while its reference count exceeds one; the
first sequence that writes a row into a shared block gets a fresh block
instead, and the block's contents are copied over (the caller runs the
queued copies, ``pa_copy_blocks``, before the writer).  The other holders
keep the original block.

"Rolling buffer cache" (llama.cpp discussion 3581, opening post): with a
window of W tokens the cache is a ring of W rows; position i goes to row
i mod W, overwriting older positions.

Sizing reading (the pages give no formula): one block of one layer holds K
and V of ``block_size`` tokens for every KV head; the block count is the
budget divided by (block bytes x layers), rounded down, with MB read as MiB.

Everything here is plain integer bookkeeping on the host.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

DEFAULT_BLOCK_SIZE = 32
CACHE_DTYPES = ("auto", "f8e4m3", "i8")
MIB = 1 << 20


@dataclass(frozen=True)
class PagedKVConfig:
    """Pool configuration, mirroring the pages' knobs.

    Exactly one of ``gpu_mem_mb`` (budget in MiB), ``gpu_mem_usage``
    (fraction of free device memory) or ``context_size`` (tokens per
    sequence-slot of the pool) sets the size.
    """

    block_size: int = DEFAULT_BLOCK_SIZE
    cache_dtype: str = "auto"
    gpu_mem_mb: Optional[int] = None
    gpu_mem_usage: Optional[float] = None
    context_size: Optional[int] = None
    window: int = 0

    def __post_init__(self):
        if self.block_size <= 0:
            raise ValueError("block_size must be positive")
        if self.cache_dtype not in CACHE_DTYPES:
            raise ValueError(f"cache_dtype must be one of {CACHE_DTYPES}")
        given = [x is not None for x in (self.gpu_mem_mb, self.gpu_mem_usage, self.context_size)]
        if sum(given) > 1:
            raise ValueError("give at most one of gpu_mem_mb, gpu_mem_usage, context_size")
        if self.gpu_mem_usage is not None and not 0 < self.gpu_mem_usage <= 1:
            raise ValueError("gpu_mem_usage must be in (0, 1]")
        if self.window < 0 or (self.window and self.window % self.block_size):
            raise ValueError("window must be a non-negative multiple of block_size")


def element_bytes(cache_dtype: str, act_bytes: int = 2) -> int:
    return 1 if cache_dtype in ("f8e4m3", "i8") else act_bytes


def bytes_per_block(cfg: PagedKVConfig, num_kv_heads: int, head_dim: int,
                    num_layers: int = 1, act_bytes: int = 2) -> int:
    """Device bytes of one block across all layers, K and V together (an INT8
    cache also keeps one fp32 scale per row and head)."""
    row = head_dim * element_bytes(cfg.cache_dtype, act_bytes)
    if cfg.cache_dtype == "i8":
        row += 4
    return 2 * cfg.block_size * num_kv_heads * row * num_layers


def num_blocks(cfg: PagedKVConfig, num_kv_heads: int, head_dim: int, num_layers: int = 1,
               act_bytes: int = 2, free_bytes: Optional[int] = None) -> int:
    """Blocks the configured budget buys (same count in every layer)."""
    per = bytes_per_block(cfg, num_kv_heads, head_dim, num_layers, act_bytes)
    if cfg.context_size is not None:
        return math.ceil(cfg.context_size / cfg.block_size)
    if cfg.gpu_mem_mb is not None:
        return (cfg.gpu_mem_mb * MIB) // per
    if cfg.gpu_mem_usage is not None:
        if free_bytes is None:
            raise ValueError("gpu_mem_usage needs the free device memory")
        return int(cfg.gpu_mem_usage * free_bytes) // per
    raise ValueError("no pool size configured")


def pool_bytes(cfg: PagedKVConfig, blocks: int, num_kv_heads: int, head_dim: int,
               num_layers: int = 1, act_bytes: int = 2) -> int:
    """Device bytes of ``blocks`` blocks in every layer (K, V and, for an
    INT8 cache, the row scales)."""
    return blocks * bytes_per_block(cfg, num_kv_heads, head_dim, num_layers, act_bytes)


class PoolTooLarge(MemoryError):
    """The pool does not fit: raised before anything is allocated (the pages
    allocate the pool up front, so an oversized budget is an out-of-memory
    error at start-up; here it is this error, with the sizes)."""


def check_pool_fits(need_bytes: int, free_bytes: Optional[int],
                    budget_bytes: Optional[int] = None) -> None:
    """Raise :class:`PoolTooLarge` when ``need_bytes`` exceeds the budget or
    the device's free memory (either may be None: not checked)."""
    if budget_bytes is not None and need_bytes > budget_bytes:
        raise PoolTooLarge(f"the KV pool needs {need_bytes / MIB:.1f} MiB, more than its "
                           f"budget of {budget_bytes / MIB:.1f} MiB")
    if free_bytes is not None and need_bytes > free_bytes:
        raise PoolTooLarge(f"the KV pool needs {need_bytes / MIB:.1f} MiB but the device has "
                           f"{free_bytes / MIB:.1f} MiB free; lower gpu_mem_mb / gpu_mem_usage "
                           f"or the context size")


def plan_pool(cfg: PagedKVConfig, num_kv_heads: int, head_dim: int, num_layers: int = 1,
              act_bytes: int = 2, free_bytes: Optional[int] = None) -> int:
    """Blocks per layer for ``cfg``, checked against the budget and the free
    memory before any allocation; raises :class:`PoolTooLarge`."""
    n = num_blocks(cfg, num_kv_heads, head_dim, num_layers, act_bytes, free_bytes)
    if n < 1:
        raise PoolTooLarge("the budget does not hold one block of every layer")
    budget = None
    if cfg.gpu_mem_mb is not None:
        budget = cfg.gpu_mem_mb * MIB
    elif cfg.gpu_mem_usage is not None:
        budget = int(cfg.gpu_mem_usage * free_bytes)
    check_pool_fits(pool_bytes(cfg, n, num_kv_heads, head_dim, num_layers, act_bytes),
                    free_bytes, budget)
    return n


class OutOfBlocks(RuntimeError):
    pass


class BlockAllocator:
    """Free list of physical block ids with reference counts.

    A block shared by several sequences (a cached prefix) is freed when its
    last holder releases it.
    """

    def __init__(self, num_blocks: int, order: Optional[Sequence[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = num_blocks
        ids = list(range(num_blocks)) if order is None else [int(i) for i in order]
        if sorted(ids) != list(range(num_blocks)):
            raise ValueError("order must be a permutation of the block ids")
        self._free: List[int] = ids[::-1]          # pop() hands out ids in `order`
        self._ref = np.zeros(num_blocks, dtype=np.int64)

    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise OutOfBlocks("KV block pool exhausted")
        blk = self._free.pop()
        self._ref[blk] = 1
        return blk

    def share(self, blk: int) -> int:
        if self._ref[blk] <= 0:
            raise ValueError(f"block {blk} is not allocated")
        self._ref[blk] += 1
        return blk

    def release(self, blk: int) -> None:
        if self._ref[blk] <= 0:
            raise ValueError(f"block {blk} is not allocated")
        self._ref[blk] -= 1
        if self._ref[blk] == 0:
            self._free.append(blk)

    def refcount(self, blk: int) -> int:
        return int(self._ref[blk])


class SequenceBlocks:
    """Blocks of one sequence: logical block j -> physical block ``blocks[j]``.

    Full cache: position p lives in logical row p.  Rolling buffer (window W):
    position p lives in ring row p mod W, and the sequence owns exactly W/BS
    blocks once it has reached W tokens.
    """

    def __init__(self, allocator: BlockAllocator, block_size: int, window: int = 0):
        self.alloc = allocator
        self.bs = block_size
        self.window = window
        self.blocks: List[int] = []
        self.num_tokens = 0
        self.pending_copies: List[tuple] = []   # (src, dst) block copies to run

    def _row(self, pos: int) -> int:
        return pos % self.window if self.window else pos

    def _ensure_row(self, row: int) -> None:
        while row // self.bs >= len(self.blocks):
            self.blocks.append(self.alloc.allocate())

    def slot(self, pos: int) -> int:
        """Flat cache slot of absolute position ``pos`` (must be resident)."""
        row = self._row(pos)
        return self.blocks[row // self.bs] * self.bs + row % self.bs

    def _writable(self, j: int) -> None:
        """Copy-on-write: make logical block j private before a row of it is
        written (queues the copy of the shared contents)."""
        blk = self.blocks[j]
        if self.alloc.refcount(blk) > 1:
            fresh = self.alloc.allocate()
            self.pending_copies.append((blk, fresh))
            self.alloc.release(blk)
            self.blocks[j] = fresh

    def append(self, n: int = 1) -> List[int]:
        """Reserve the next ``n`` positions; returns their slots.  Writing
        into a shared block first gives this sequence its own copy (see
        :meth:`take_copies`).  Rolling buffer: a position that a later one
        of the same call overwrites gets slot -1 (the writer skips it), so
        no two tokens of one write share a ring row."""
        end = self.num_tokens + n
        out = []
        for _ in range(n):
            pos = self.num_tokens
            row = self._row(pos)
            self._ensure_row(row)
            self._writable(row // self.bs)
            self.num_tokens += 1
            lands = not self.window or pos >= end - self.window
            out.append(self.slot(pos) if lands else -1)
        return out

    def take_copies(self) -> np.ndarray:
        """The queued (src, dst) block copies as ``[N, 2]`` int32, cleared.
        Run them (``ops.copy_blocks``) before writing the reserved slots."""
        out = np.array(self.pending_copies, dtype=np.int32).reshape(-1, 2)
        self.pending_copies = []
        return out

    def share_prefix(self, other: "SequenceBlocks", num_tokens: int) -> None:
        """Start this (empty) sequence with ``other``'s first ``num_tokens``
        positions by sharing the blocks that hold them, a partially filled
        last block included (it is copied when either side writes to it)."""
        if self.blocks or self.num_tokens:
            raise ValueError("share_prefix needs an empty sequence")
        if self.window or other.window:
            raise ValueError("shared prefixes are for full caches")
        if num_tokens > other.num_tokens:
            raise ValueError("prefix must be resident in the other sequence")
        for blk in other.blocks[: -(-num_tokens // self.bs)]:
            self.blocks.append(self.alloc.share(blk))
        self.num_tokens = num_tokens

    def fork(self) -> "SequenceBlocks":
        """A new sequence sharing all of this one's positions."""
        child = SequenceBlocks(self.alloc, self.bs, self.window)
        child.share_prefix(self, self.num_tokens)
        return child

    def context_len(self) -> int:
        return self.num_tokens

    def release(self) -> None:
        for blk in self.blocks:
            self.alloc.release(blk)
        self.blocks = []
        self.num_tokens = 0


class MixedLayerKV:
    """Block bookkeeping of a model whose layers are full-attention or
    sliding-window ("libmir-metal 0.2.0, src/native/trace/kv.rs", fn build:
    full-attention layers keep paged K/V, sliding layers a bounded ring, the
    pages keyed by layer and session).

    ``layer_windows[l]`` is 0 for a full layer, else its window W (a multiple
    of the block size).  Layers with the same window advance together, so
    they share one allocator, one table and one slot mapping per sequence
    (a group); each layer keeps its own K/V pools of its group's block
    count.  ``blocks`` maps a window to the pool size of its group.
    """

    def __init__(self, layer_windows: Sequence[int], block_size: int,
                 blocks: Dict[int, int]):
        self.layer_windows = [int(w) for w in layer_windows]
        self.bs = block_size
        self.windows = sorted(set(self.layer_windows))
        for w in self.windows:
            if w < 0 or (w and w % block_size):
                raise ValueError("windows must be 0 or positive multiples of block_size")
            if w not in blocks:
                raise ValueError(f"no pool size for window {w}")
        self.alloc = {w: BlockAllocator(int(blocks[w])) for w in self.windows}
        self.seqs: Dict[object, Dict[int, SequenceBlocks]] = {}

    def add(self, seq_id) -> None:
        if seq_id in self.seqs:
            raise ValueError(f"sequence {seq_id!r} exists")
        self.seqs[seq_id] = {w: SequenceBlocks(self.alloc[w], self.bs, w) for w in self.windows}

    def release(self, seq_id) -> None:
        for s in self.seqs.pop(seq_id).values():
            s.release()

    def append(self, seq_id, n: int) -> Dict[int, List[int]]:
        """Reserve the next ``n`` positions in every group; slots per window
        (a ring's overwritten-within-the-call positions get -1)."""
        return {w: s.append(n) for w, s in self.seqs[seq_id].items()}

    def num_tokens(self, seq_id) -> int:
        return self.seqs[seq_id][self.windows[0]].num_tokens

    def max_blocks(self, window: int, max_context: int) -> int:
        """Table width of a group: the ring's W / BS, or enough for max_context."""
        return window // self.bs if window else -(-max_context // self.bs)

    def tables(self, seq_ids: Sequence, window: int, max_blocks: int) -> np.ndarray:
        """``[B, max_blocks]`` int32 tables of one group."""
        return block_table_array([self.seqs[i][window] for i in seq_ids], max_blocks)

    def context_lens(self, seq_ids: Sequence) -> np.ndarray:
        return np.array([self.num_tokens(i) for i in seq_ids], dtype=np.int32)


def block_table_array(seqs: Sequence[SequenceBlocks], max_blocks: Optional[int] = None,
                      pad: int = 0) -> np.ndarray:
    """``[B, MBPS]`` int32 block tables, padded with ``pad``."""
    mbps = max_blocks or max(1, max(len(s.blocks) for s in seqs))
    bt = np.full((len(seqs), mbps), pad, dtype=np.int32)
    for b, s in enumerate(seqs):
        if len(s.blocks) > mbps:
            raise ValueError("sequence has more blocks than max_blocks")
        bt[b, : len(s.blocks)] = s.blocks
    return bt


def identity_table(B: int, max_blocks: int) -> np.ndarray:
    """Block tables of a dense pool: sequence b owns physical blocks
    ``b * max_blocks .. (b + 1) * max_blocks - 1`` in order.  The attention
    entry points take such a map without a table (``ops.IdentityMap``)."""
    return (np.arange(B, dtype=np.int64)[:, None] * max_blocks
            + np.arange(max_blocks, dtype=np.int64)[None, :]).astype(np.int32)


def is_identity(block_tables: np.ndarray, context_lens: Optional[np.ndarray] = None,
                block_size: int = DEFAULT_BLOCK_SIZE) -> bool:
    """True when every table entry the kernels read is the identity map:
    the first ``ceil(context_lens[b] / block_size)`` entries of row b (all of
    them without ``context_lens``) equal ``b * MBPS + j``."""
    bt = np.asarray(block_tables)
    ident = identity_table(bt.shape[0], bt.shape[1])
    if context_lens is None:
        return bool(np.array_equal(bt, ident))
    for b, L in enumerate(np.asarray(context_lens)):
        n = min(-(-int(L) // block_size), bt.shape[1])
        if not np.array_equal(bt[b, :n], ident[b, :n]):
            return False
    return True


def slots_from_table(block_table_row: np.ndarray, positions: np.ndarray, block_size: int,
                     window: int = 0) -> np.ndarray:
    """Vectorised slot mapping of absolute positions through one table row."""
    pos = np.asarray(positions, dtype=np.int64)
    rows = pos % window if window else pos
    phys = np.asarray(block_table_row, dtype=np.int64)[rows // block_size]
    return (phys * block_size + rows % block_size).astype(np.int32)


def describe(cfg: PagedKVConfig, num_layers: int, cached_tokens: int) -> Dict[str, object]:
    """Cache description in the shape of a trace record (dtype, block size,
    page key, prefix cache, counts), as the libmir-metal trace builder reports."""
    return {
        "dtype": cfg.cache_dtype,
        "quant_mode": {"f8e4m3": "per-tensor fp32 scale",
                       "i8": "per-token/head fp32 scale"}.get(cfg.cache_dtype, "none"),
        "decode_attention": "paged split-context decode (HIP, gfx950)",
        "block_size": cfg.block_size,
        "physical_page_key": "layer + sequence; head-major pages"
        + ("; rolling ring" if cfg.window else "")
        + ("; packed INT8 pages and per-token/head fp32 scales" if cfg.cache_dtype == "i8"
           else ""),
        "paged_attention": True,
        "entry_count": num_layers,
        "cached_tokens": cached_tokens,
        "resident_token_slots": cached_tokens,
    }
