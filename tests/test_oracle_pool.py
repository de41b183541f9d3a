"""Pins for the oracle's pool sizing and ring rule against the pages' numbers.

Fixtures in ``tests/golden/`` carry their citations.
"""

import json
import os

from oracle import pool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_default_block_size():
    g = _golden("pages_numbers.json")
    assert pool.DEFAULT_BLOCK_SIZE == g["default_block_size"]["value"]


def test_rolling_buffer_memory_ratio_at_32k():
    g = _golden("pages_numbers.json")["rolling_buffer_reduction"]
    seq, W, BS = g["sequence_length"], g["window"], g["block_size"]
    full_blocks = pool.blocks_for_context(seq, BS)
    ring_blocks = pool.blocks_for_context(W, BS)
    assert full_blocks == 1024 and ring_blocks == 128
    assert full_blocks // ring_blocks == g["reduction"]
    assert full_blocks % ring_blocks == 0


def test_fp8_halves_memory():
    g = _golden("pages_numbers.json")["fp8_vs_fp16"]
    # Mistral-7B shape (8 KV heads, head_dim 128, 32 layers) at the pages'
    # 4096 MiB budget.
    n16 = pool.blocks_for_mib(g["budget_mib"], 32, 8, 128, "f16", num_layers=32)
    n8 = pool.blocks_for_mib(g["budget_mib"], 32, 8, 128, "e4m3", num_layers=32)
    assert n16 == 1024 and n8 == 2048
    assert n8 == 2 * n16
    # Inexact budgets: within one block of twice.
    for mib in (1000, 4095, 8191, 12345):
        a = pool.blocks_for_mib(mib, 32, 8, 128, "f16", 32)
        b = pool.blocks_for_mib(mib, 32, 8, 128, "e4m3", 32)
        assert 2 * a <= b <= 2 * a + 1


def test_block_bytes_closed_form():
    # One block of 32 tokens, 8 heads x 128 dims, bf16, K and V: 2*32*8*128*2.
    assert pool.block_bytes(32, 8, 128, "bf16") == 131072
    assert pool.block_bytes(32, 8, 128, "e4m3") == 65536


def test_context_size_and_fraction():
    # ContextSize(1024) with block size 32 (the Rust API example) -> 32 blocks.
    assert pool.blocks_for_context(1024, 32) == 32
    assert pool.blocks_for_context(1025, 32) == 33
    free = 10 * (1 << 30)
    n = pool.blocks_for_fraction(0.95, free, 32, 8, 128, "bf16")
    assert n == int(0.95 * free) // 131072


def test_ring_w3_worked_example():
    g = _golden("rolling_buffer_w3.json")
    held = pool.positions_in_ring(g["last_position"], g["window"])
    assert {str(k): v for k, v in held.items()} == g["ring_contents"]
