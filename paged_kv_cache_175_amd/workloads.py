"""Seeded synthetic inputs for the paged KV-cache path.

This module only draws random inputs and lays them out; it holds none of the
method's arithmetic (no slot arithmetic, no encoding, no attention).  Both the
HIP path and the CPU oracle consume what it returns, each with its own code.

Values are fp32 standard normals rounded (RNE, by torch's cast) to the
activation dtype.  The workloads are shaped like the chat runs the pages
describe ("PagedAttention in mistral.rs": Mistral-7B-Instruct and
Phi-3-mini examples with block size 32; "Rolling buffer cache", llama.cpp
discussion 3581: Mistral-7B's 4096-token window at 32k positions).  No model
weights or datasets are involved.

Draw order for every workload, from one ``numpy.random.default_rng(seed)``:

1. context lengths (or absolute positions);
2. a permutation of the physical blocks, sliced in sequence order into the
   block tables;
3. the query;
4. per-sequence K/V of the cached tokens, in position order;
5. K/V of the new tokens.

Pools get one extra block at index ``num_blocks`` (the *poison* block).  Table
entries past a sequence's last block point at it, and pools start filled with
NaN, so any read outside the live rows shows up as NaN in the output.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BLOCK_SIZE = 32

_TORCH_ACT = {"bf16": torch.bfloat16, "f16": torch.float16}


def to_act_bits(x_f32: np.ndarray, act: str) -> np.ndarray:
    """RNE-round fp32 values to ``act`` (bf16 or f16) and return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(_TORCH_ACT[act]).view(torch.int16).numpy().view(np.uint16)


def act_bits_to_f32(bits: np.ndarray, act: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(_TORCH_ACT[act]).to(torch.float32).numpy()


def _normal_bits(rng, shape, act):
    return to_act_bits(rng.standard_normal(shape, dtype=np.float32), act)


def _amax_scale(bits_list, act) -> float:
    """Per-tensor fp32 scale amax/448 over every generated value."""
    amax = np.float32(0.0)
    for bits in bits_list:
        if bits.size:
            amax = max(amax, np.float32(np.max(np.abs(act_bits_to_f32(bits, act)))))
    return float(np.float32(amax) / np.float32(448.0))


@dataclass
class DecodeWorkload:
    """One decode step of a batch of sequences.

    Cached tokens of sequence b: ``cached_k[b]`` / ``cached_v[b]`` with shape
    ``[n_cached_b, Hkv, D]`` in position order starting at ``cached_pos0[b]``.
    New token of sequence b: ``new_k[b]`` / ``new_v[b]`` at position
    ``new_pos[b]``.  ``context_lens[b] = new_pos[b] + 1`` (absolute position of
    the decoded token plus one).  With ``window > 0`` the table addresses a
    ring of ``window`` rows.
    """

    name: str
    act: str
    cache: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    num_blocks: int            # live blocks; the poison block is num_blocks
    max_blocks_per_seq: int
    scale: float
    window: int
    context_lens: np.ndarray   # int32 [B]
    block_tables: np.ndarray   # int32 [B, MBPS]
    query: np.ndarray          # uint16 [B, Hq, D]
    cached_pos0: np.ndarray    # int64 [B]
    cached_k: list             # B x uint16 [n, Hkv, D]
    cached_v: list
    new_pos: np.ndarray        # int64 [B]
    new_k: np.ndarray          # uint16 [B, Hkv, D]
    new_v: np.ndarray
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def poison_block(self) -> int:
        return self.num_blocks

    @property
    def pool_blocks(self) -> int:
        return self.num_blocks + 1

    def kv_read_tokens(self) -> int:
        """Tokens the decode reads, summed over sequences (per KV head)."""
        L = self.context_lens.astype(np.int64)
        if self.window > 0:
            L = np.minimum(L, self.window)
        return int(L.sum())


def _tables_from_perm(perm, blocks_per_seq, mbps, poison):
    B = len(blocks_per_seq)
    bt = np.full((B, mbps), poison, dtype=np.int32)
    off = 0
    for b, nb in enumerate(blocks_per_seq):
        bt[b, :nb] = perm[off:off + nb]
        off += nb
    return bt


def decode_workload(name: str, seed: int, B: int, Hq: int, Hkv: int, D: int,
                    act: str, cache: Optional[str] = None, ctx: Optional[list] = None,
                    ctx_range: Optional[tuple] = None, window: int = 0,
                    pos_range: Optional[tuple] = None, num_blocks: Optional[int] = None,
                    max_blocks_per_seq: Optional[int] = None,
                    BS: int = BLOCK_SIZE) -> DecodeWorkload:
    """Build a decode workload.

    Full cache (window == 0): context lengths come from ``ctx`` or are drawn
    uniformly from ``ctx_range`` (inclusive); each sequence gets
    ceil(ctx/BS) blocks.  ``num_blocks`` defaults to the total needed.

    Rolling buffer (window > 0): absolute positions of the decoded token are
    drawn uniformly from ``pos_range`` (inclusive); each sequence owns
    window/BS blocks; the cached tokens are the ``min(pos, window)`` positions
    before the decoded one.
    """
    cache = cache or act
    rng = np.random.default_rng(seed)
    # 1. lengths / positions
    if window > 0:
        lo, hi = pos_range
        pos = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        blocks_per_seq = [window // BS] * B
    else:
        if ctx is not None:
            L = np.asarray(ctx, dtype=np.int64)
        else:
            lo, hi = ctx_range
            L = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        pos = L - 1
        blocks_per_seq = [int(-(-int(l) // BS)) for l in L]
    total_blocks = int(sum(blocks_per_seq))
    nb = num_blocks if num_blocks is not None else total_blocks
    if nb < total_blocks:
        raise ValueError("pool too small for the drawn contexts")
    mbps = max_blocks_per_seq or max(blocks_per_seq)
    # 2. permutation -> tables (padding points at the poison block nb)
    perm = rng.permutation(nb).astype(np.int32)
    bt = _tables_from_perm(perm, blocks_per_seq, mbps, nb)
    # 3. query
    q = _normal_bits(rng, (B, Hq, D), act)
    # 4. cached tokens, position order
    ck, cv, pos0 = [], [], np.zeros(B, dtype=np.int64)
    for b in range(B):
        if window > 0:
            n = int(min(pos[b], window))
        else:
            n = int(pos[b])
        pos0[b] = pos[b] - n
        ck.append(_normal_bits(rng, (n, Hkv, D), act))
        cv.append(_normal_bits(rng, (n, Hkv, D), act))
    # 5. new tokens
    nk = _normal_bits(rng, (B, Hkv, D), act)
    nv = _normal_bits(rng, (B, Hkv, D), act)
    k_scale = v_scale = 1.0
    if cache == "e4m3":
        k_scale = _amax_scale(ck + [nk], act)
        v_scale = _amax_scale(cv + [nv], act)
    return DecodeWorkload(
        name=name, act=act, cache=cache, B=B, Hq=Hq, Hkv=Hkv, D=D, BS=BS,
        num_blocks=nb, max_blocks_per_seq=mbps, scale=float(1.0 / np.sqrt(D)),
        window=window, context_lens=(pos + 1).astype(np.int32), block_tables=bt,
        query=q, cached_pos0=pos0, cached_k=ck, cached_v=cv, new_pos=pos,
        new_k=nk, new_v=nv, k_scale=k_scale, v_scale=v_scale,
        meta={"seed": seed})


@dataclass
class PrefillWorkload:
    """Chunked prefill: each sequence appends a chunk after a shared prefix.

    The prefix K/V (``prefix_k``/``prefix_v``, ``[P, Hkv, D]``) occupies the
    same physical blocks (``shared_blocks``) in every table; chunk b's K/V
    (``chunk_k[b]``) goes to that sequence's private blocks.
    """

    name: str
    act: str
    cache: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    prefix_len: int
    chunk_lens: np.ndarray     # int32 [B]
    cu_q_lens: np.ndarray      # int32 [B+1]
    context_lens: np.ndarray   # int32 [B] = prefix + chunk
    block_tables: np.ndarray   # int32 [B, MBPS]
    shared_blocks: np.ndarray  # int32 [prefix_len / BS]
    query: np.ndarray          # uint16 [total_q, Hq, D]
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    chunk_k: list              # B x uint16 [C_b, Hkv, D]
    chunk_v: list
    k_scale: float = 1.0
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    @property
    def poison_block(self) -> int:
        return self.num_blocks

    @property
    def pool_blocks(self) -> int:
        return self.num_blocks + 1

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    def flops(self) -> int:
        """Causal attention FLOPs: 4*D per (query, visible key) pair per head."""
        n = 0
        for b in range(self.B):
            C = int(self.chunk_lens[b])
            ctx = int(self.context_lens[b])
            first = ctx - C + 1
            n += C * first + C * (C - 1) // 2
        return 4 * self.D * self.Hq * n


def prefill_workload(name: str, seed: int, B: int, Hq: int, Hkv: int, D: int,
                     act: str, prefix_len: int, chunk: Optional[int] = None,
                     chunk_range: Optional[tuple] = None, cache: Optional[str] = None,
                     BS: int = BLOCK_SIZE, chunks: Optional[list] = None) -> PrefillWorkload:
    """Build a chunked-prefill workload over a shared prefix.

    ``prefix_len`` must be a multiple of BS (whole shared blocks).  Chunk
    lengths are ``chunk`` for every sequence, the list ``chunks``, or drawn
    from ``chunk_range``.
    """
    if prefix_len % BS:
        raise ValueError("prefix must be whole blocks")
    cache = cache or act
    rng = np.random.default_rng(seed)
    # 1. lengths
    if chunks is not None:
        C = np.asarray(chunks, dtype=np.int64)
        if C.shape != (B,):
            raise ValueError("chunks must list B lengths")
    elif chunk is not None:
        C = np.full(B, chunk, dtype=np.int64)
    else:
        lo, hi = chunk_range
        C = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    n_shared = prefix_len // BS
    priv = [int(-(-int(c) // BS)) for c in C]
    nb = n_shared + sum(priv)
    mbps = n_shared + max(priv)
    # 2. permutation: first the shared blocks, then private blocks in order
    perm = rng.permutation(nb).astype(np.int32)
    shared = perm[:n_shared].copy()
    bt = np.full((B, mbps), nb, dtype=np.int32)
    off = n_shared
    for b in range(B):
        bt[b, :n_shared] = shared
        bt[b, n_shared:n_shared + priv[b]] = perm[off:off + priv[b]]
        off += priv[b]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(C)
    # 3. query
    q = _normal_bits(rng, (int(cu[-1]), Hq, D), act)
    # 4. cached (prefix) tokens
    pk = _normal_bits(rng, (prefix_len, Hkv, D), act)
    pv = _normal_bits(rng, (prefix_len, Hkv, D), act)
    # 5. new (chunk) tokens
    ck = [_normal_bits(rng, (int(c), Hkv, D), act) for c in C]
    cv = [_normal_bits(rng, (int(c), Hkv, D), act) for c in C]
    k_scale = v_scale = 1.0
    if cache == "e4m3":
        k_scale = _amax_scale([pk] + ck, act)
        v_scale = _amax_scale([pv] + cv, act)
    return PrefillWorkload(
        name=name, act=act, cache=cache, B=B, Hq=Hq, Hkv=Hkv, D=D, BS=BS,
        num_blocks=nb, max_blocks_per_seq=mbps, scale=float(1.0 / np.sqrt(D)),
        prefix_len=prefix_len, chunk_lens=C.astype(np.int32), cu_q_lens=cu,
        context_lens=(prefix_len + C).astype(np.int32), block_tables=bt,
        shared_blocks=shared, query=q, prefix_k=pk, prefix_v=pv, chunk_k=ck,
        chunk_v=cv, k_scale=k_scale, v_scale=v_scale, meta={"seed": seed})


@dataclass
class WindowPrefillWorkload:
    """Chunked prefill of a sliding-window layer whose cache is a ring.

    Sequence b has ``hist_lens[b]`` positions before its chunk; the ring
    (``window / BS`` blocks, table row b) holds the last ``min(hist, W)`` of
    them, positions ``hist_pos0[b]`` .. ``hist_lens[b] - 1`` with K/V
    ``hist_k[b]`` / ``hist_v[b]``.  The chunk's K/V ``chunk_k`` /
    ``chunk_v`` ``[total_q, Hkv, D]`` are packed like the queries.
    """

    name: str
    act: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    window: int
    num_blocks: int
    scale: float
    hist_lens: np.ndarray      # int32 [B]
    hist_pos0: np.ndarray      # int32 [B] first position still in the ring
    chunk_lens: np.ndarray     # int32 [B]
    cu_q_lens: np.ndarray      # int32 [B+1]
    context_lens: np.ndarray   # int32 [B] = hist + chunk
    block_tables: np.ndarray   # int32 [B, window / BS]
    query: np.ndarray          # uint16 [total_q, Hq, D]
    chunk_k: np.ndarray        # uint16 [total_q, Hkv, D]
    chunk_v: np.ndarray
    hist_k: list               # B x uint16 [hist - hist_pos0, Hkv, D]
    hist_v: list
    cache: str = ""
    k_scale: float = 1.0       # 16-bit ring: no quantisation scales
    v_scale: float = 1.0
    meta: dict = field(default_factory=dict)

    def __post_init__(self):
        self.cache = self.cache or self.act

    @property
    def pool_blocks(self) -> int:
        return self.num_blocks

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1])

    def flops(self) -> int:
        """4*D per (query, visible key) pair per head; query i sees min(i+1, W) keys."""
        n = 0
        for b in range(self.B):
            h, C = int(self.hist_lens[b]), int(self.chunk_lens[b])
            i = np.arange(h, h + C, dtype=np.int64)
            n += int(np.minimum(i + 1, self.window).sum())
        return 4 * self.D * self.Hq * n


def window_prefill_workload(name: str, seed: int, B: int, Hq: int, Hkv: int, D: int,
                            act: str, window: int, hist, chunk, BS: int = BLOCK_SIZE,
                            cache: Optional[str] = None) -> WindowPrefillWorkload:
    """Build a sliding-window chunked-prefill workload.

    ``hist`` / ``chunk``: one length for every sequence, a list of B
    lengths, or a (lo, hi) range to draw from (a tuple).  The B rings take
    distinct blocks of one shuffled pool.  ``cache``: the ring's format (the
    activation format by default; "e4m3" gets per-tensor scales amax / 448
    over the history and the chunk, "int8" quantises per row when written).
    """
    if window <= 0 or window % BS:
        raise ValueError("window must be a positive multiple of the block size")
    rng = np.random.default_rng(seed)

    def lengths(spec):
        if isinstance(spec, tuple):
            return rng.integers(spec[0], spec[1] + 1, size=B).astype(np.int64)
        if np.isscalar(spec):
            return np.full(B, int(spec), dtype=np.int64)
        return np.asarray(spec, dtype=np.int64)

    H = lengths(hist)
    C = lengths(chunk)
    nblk = window // BS
    nb = B * nblk
    bt = rng.permutation(nb).astype(np.int32).reshape(B, nblk)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(C)
    pos0 = np.maximum(H - window, 0)
    q = _normal_bits(rng, (int(cu[-1]), Hq, D), act)
    ck = _normal_bits(rng, (int(cu[-1]), Hkv, D), act)
    cv = _normal_bits(rng, (int(cu[-1]), Hkv, D), act)
    hk = [_normal_bits(rng, (int(h - p), Hkv, D), act) for h, p in zip(H, pos0)]
    hv = [_normal_bits(rng, (int(h - p), Hkv, D), act) for h, p in zip(H, pos0)]
    k_scale = v_scale = 1.0
    if cache == "e4m3":
        k_scale = _amax_scale(hk + [ck], act)
        v_scale = _amax_scale(hv + [cv], act)
    return WindowPrefillWorkload(
        name=name, act=act, B=B, Hq=Hq, Hkv=Hkv, D=D, BS=BS, window=window, num_blocks=nb,
        scale=float(1.0 / np.sqrt(D)), hist_lens=H.astype(np.int32),
        hist_pos0=pos0.astype(np.int32), chunk_lens=C.astype(np.int32), cu_q_lens=cu,
        context_lens=(H + C).astype(np.int32), block_tables=bt, query=q, chunk_k=ck,
        chunk_v=cv, hist_k=hk, hist_v=hv, cache=cache or act, k_scale=k_scale,
        v_scale=v_scale, meta={"seed": seed})


# ---------------------------------------------------------------------------
# The five named workloads.


def tiny_decode() -> DecodeWorkload:
    """2 sequences (contexts 37 and 64), 4/4 heads, head_dim 64, fp16, 16 blocks."""
    return decode_workload("tiny_decode", seed=0, B=2, Hq=4, Hkv=4, D=64, act="f16",
                           ctx=[37, 64], num_blocks=16)


def mistral_decode(B: int = 32, ctx_range=(512, 4096), seed: int = 1) -> DecodeWorkload:
    """Mistral-7B-shaped decode: 32/8 heads, head_dim 128, bf16."""
    return decode_workload("mistral_decode", seed=seed, B=B, Hq=32, Hkv=8, D=128,
                           act="bf16", ctx_range=ctx_range)


def fp8_decode(B: int = 64, ctx_range=(1024, 8192), seed: int = 2) -> DecodeWorkload:
    """Mistral-7B decode shape with an E4M3 cache (per-tensor amax/448 scales)."""
    return decode_workload("fp8_decode", seed=seed, B=B, Hq=32, Hkv=8, D=128,
                           act="bf16", cache="e4m3", ctx_range=ctx_range)


def int8_decode(B: int = 64, ctx_range=(1024, 8192), seed: int = 5) -> DecodeWorkload:
    """The FP8 decode shape with an INT8 per-token/head cache (fp32 row scales)."""
    return decode_workload("int8_decode", seed=seed, B=B, Hq=32, Hkv=8, D=128, act="bf16",
                           cache="int8", ctx_range=ctx_range)


def sliding_decode(B: int = 8, window: int = 4096, pos_range=(4096, 32768),
                   seed: int = 3) -> DecodeWorkload:
    """Rolling-buffer decode: W-row ring per sequence, 32/8 heads, head_dim 128."""
    return decode_workload("sliding_decode", seed=seed, B=B, Hq=32, Hkv=8, D=128,
                           act="bf16", window=window, pos_range=pos_range)


def sliding_prefill(B: int = 4, window: int = 4096, hist: int = 8192, chunk: int = 2048,
                    seed: int = 6, cache: Optional[str] = None) -> WindowPrefillWorkload:
    """Mistral-7B-shaped sliding-window layer (32/8 heads, head_dim 128, bf16,
    4096-token window): chunks of 2048 tokens after 8192 positions, so the
    ring is full and every query sees 4096 keys.  ``cache``: "e4m3" or
    "int8" for a quantised ring (named sliding_prefill_fp8 / _int8)."""
    name = {None: "sliding_prefill", "e4m3": "sliding_prefill_fp8",
            "int8": "sliding_prefill_int8"}[cache]
    return window_prefill_workload(name, seed, B=B, Hq=32, Hkv=8, D=128, act="bf16",
                                   window=window, hist=hist, chunk=chunk, cache=cache)


@dataclass
class CopyWorkload:
    """A burst of copy-on-write block copies: ``mapping`` ``[N, 2]`` (src,
    dst) over a pool of ``num_blocks`` blocks, distinct blocks throughout."""

    name: str
    cache: str
    Hkv: int
    D: int
    BS: int
    num_blocks: int
    mapping: np.ndarray        # int32 [N, 2]
    meta: dict = field(default_factory=dict)

    def block_bytes(self) -> int:
        elem = {"e4m3": 1, "int8": 1}.get(self.cache, 2)
        row = self.D * elem + (4 if self.cache == "int8" else 0)
        return 2 * self.Hkv * self.BS * row


def cow_copy(N: int = 2048, seed: int = 7) -> CopyWorkload:
    """Copy-on-write after forks, Mistral-7B layer shape (8 KV heads,
    head_dim 128, bf16 cache, 128 KiB per block): 2048 copies, e.g. 64
    forked sequences each copying the shared partial last block of 32
    layers, from and to random distinct blocks of a 4096-block pool."""
    rng = np.random.default_rng(seed)
    nb = 2 * N
    perm = rng.permutation(nb).astype(np.int32)
    return CopyWorkload(name="cow_copy", cache="bf16", Hkv=8, D=128, BS=BLOCK_SIZE,
                        num_blocks=nb, mapping=np.stack([perm[:N], perm[N:]], axis=1),
                        meta={"seed": seed})


def prefix_prefill(B: int = 16, prefix_len: int = 2048, chunk: int = 512,
                   seed: int = 4) -> PrefillWorkload:
    """Phi-3-mini-shaped chunked prefill over a shared prefix: 32/32 heads, D=96."""
    return prefill_workload("prefix_prefill", seed=seed, B=B, Hq=32, Hkv=32, D=96,
                            act="bf16", prefix_len=prefix_len, chunk=chunk)
