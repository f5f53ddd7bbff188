"""Oracle index metadata: what the runner hands to the store and attention calls.

TEST INFRASTRUCTURE ONLY (see the package docstring). Written from "Nano-vLLM Field Guide",
Step 05.1 (the slot of a position), Step 07.5 (packing a prefill batch), Step 07.6 (a decode
row) and Step 07.7 (block tables padded with -1), in plain Python, one position at a time.

Each sequence is given as an object with ``block_table`` (physical ids in logical order),
``num_cached`` (tokens already in the cache) and ``num_new`` (tokens computed this step).
"""
from __future__ import annotations

import numpy as np


def slot_of(block_table, position: int, block_size: int) -> int:
    """Pool row of a logical position: block id of its logical block times the block size,
    plus its offset inside the block."""
    return block_table[position // block_size] * block_size + position % block_size


def prepare_block_tables(tables) -> np.ndarray:
    """Pad every table with -1 to the longest one; int32 [B, max_len]."""
    width = max((len(t) for t in tables), default=0)
    out = np.full((len(tables), width), -1, dtype=np.int32)
    for b, t in enumerate(tables):
        out[b, :len(t)] = t
    return out


def prepare_prefill(seqs, block_size: int) -> dict:
    """New tokens of every sequence packed into one run.

    Sequence b computes positions [start, end) with start = num_cached and end = start +
    num_new; its queries are the new tokens and its keys are all `end` tokens (cached prefix
    plus new). cu_seqlens_q / cu_seqlens_k are running sums of num_new and of end.
    """
    positions, slots = [], []
    cu_q, cu_k = [0], [0]
    for s in seqs:
        start, end = s.num_cached, s.num_cached + s.num_new
        for p in range(start, end):
            positions.append(p)
            slots.append(slot_of(s.block_table, p, block_size))
        cu_q.append(cu_q[-1] + (end - start))
        cu_k.append(cu_k[-1] + end)
    q_lens = [s.num_new for s in seqs]
    k_lens = [s.num_cached + s.num_new for s in seqs]
    return dict(
        positions=np.array(positions, dtype=np.int64),
        slot_mapping=np.array(slots, dtype=np.int32),
        cu_seqlens_q=np.array(cu_q, dtype=np.int32),
        cu_seqlens_k=np.array(cu_k, dtype=np.int32),
        max_seqlen_q=max(q_lens, default=0),
        max_seqlen_k=max(k_lens, default=0),
        has_cached_context=cu_k[-1] > cu_q[-1],
        block_tables=prepare_block_tables([s.block_table for s in seqs]),
    )


def prepare_decode(seqs, block_size: int) -> dict:
    """One row per sequence: the token at position len - 1 is stored and attends to all len
    tokens. A padding row (no tokens) gets slot -1 and context length 0."""
    positions, slots, ctx = [], [], []
    for s in seqs:
        n = s.num_cached + s.num_new
        if n == 0:
            positions.append(0)
            slots.append(-1)
            ctx.append(0)
            continue
        positions.append(n - 1)
        slots.append(slot_of(s.block_table, n - 1, block_size))
        ctx.append(n)
    return dict(
        positions=np.array(positions, dtype=np.int64),
        slot_mapping=np.array(slots, dtype=np.int32),
        context_lens=np.array(ctx, dtype=np.int32),
        block_tables=prepare_block_tables([s.block_table for s in seqs]),
    )
