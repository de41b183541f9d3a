"""Pool sizing and the rolling-buffer slot rule -- test oracle.

Test infrastructure only (see the package docstring).

"PagedAttention in mistral.rs" says the pool has two inputs, a GPU memory
budget in MB and a block size in tokens (default 32), that the budget can also
be given as a fraction of GPU memory or, in the Rust API, as a context size in
tokens, and that the F8E4M3 cache type about halves the memory of an FP16
cache.  The exact sizing formula is not given; the reading used here:

* one block of one layer holds K and V for ``block_size`` tokens of every KV
  head: ``2 * block_size * num_kv_heads * head_dim * elem_bytes`` bytes;
* ``num_blocks = floor(budget_bytes / (block_bytes * num_layers))`` with MB
  read as MiB;
* a usage fraction sets ``budget = fraction * free_bytes``;
* a context size of n tokens gives ``ceil(n / block_size)`` blocks.

"Rolling buffer cache" (llama.cpp discussion 3581, opening post): a cache of
fixed size W stores timestep i at position i mod W.
"""

from __future__ import annotations

import math

ELEM_BYTES = {"f16": 2, "bf16": 2, "e4m3": 1}
DEFAULT_BLOCK_SIZE = 32
MIB = 1 << 20


def block_bytes(block_size: int, num_kv_heads: int, head_dim: int, fmt: str) -> int:
    """Bytes of one block of one layer, K and V together."""
    return 2 * block_size * num_kv_heads * head_dim * ELEM_BYTES[fmt]


def blocks_for_budget(budget_bytes: int, block_size: int, num_kv_heads: int,
                      head_dim: int, fmt: str, num_layers: int = 1) -> int:
    per = block_bytes(block_size, num_kv_heads, head_dim, fmt) * num_layers
    return budget_bytes // per


def blocks_for_mib(mib: int, block_size: int, num_kv_heads: int, head_dim: int,
                   fmt: str, num_layers: int = 1) -> int:
    return blocks_for_budget(mib * MIB, block_size, num_kv_heads, head_dim, fmt,
                             num_layers)


def blocks_for_fraction(fraction: float, free_bytes: int, block_size: int,
                        num_kv_heads: int, head_dim: int, fmt: str,
                        num_layers: int = 1) -> int:
    return blocks_for_budget(int(fraction * free_bytes), block_size, num_kv_heads,
                             head_dim, fmt, num_layers)


def blocks_for_context(tokens: int, block_size: int) -> int:
    return math.ceil(tokens / block_size)


def ring_index(position: int, window: int) -> int:
    """Ring row that holds absolute position ``position`` in a W-row ring."""
    return position % window


def positions_in_ring(position: int, window: int):
    """Absolute positions a W-row ring holds after writing 0..position in order.

    Returns a dict ring_row -> position.
    """
    held = {}
    for p in range(position + 1):
        held[ring_index(p, window)] = p
    return held
