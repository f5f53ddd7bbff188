"""Seeded synthetic workloads for the paged-KV hot path.

This module stands in for the engine's scheduler and block manager ("Nano-vLLM Field Guide",
Steps 05-06): it decides which sequences run in a step, how many tokens each already has in
the cache and how many it adds, which physical blocks each sequence owns (a random
permutation of the pool, optionally shared between prompts with a common prefix) and how long
prompts are cut into chunks. It also draws every random value: lengths, permutations, cache
contents and the new q/k/v rows.

It derives nothing that the method computes: no slot numbers, no cumulative lengths, no
context lengths and no attention values. Both the HIP library's own metadata builder and the
oracle's take the ``Seq`` descriptions below and produce those independently.

Recipe (one seed per workload, ``numpy.random.default_rng(seed)`` for integers and
``torch.Generator().manual_seed(seed)`` for values): lengths first, then the block
permutation, then the cache contents, then the new q/k/v rows. Values are N(0, 1) drawn in
fp32 and rounded to bf16 (round-to-nearest-even, torch's conversion). Blocks that no sequence
owns hold bf16 NaN when ``poison=True`` so that any stray read shows up in the output.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BF16_NAN_BITS = 0x7FC0


@dataclass(frozen=True)
class AttnShape:
    """Attention geometry of one layer: q heads, kv heads, head dim, tokens per block."""

    num_heads: int
    num_kv_heads: int
    head_dim: int = 128
    block_size: int = 256

    @property
    def row_elems(self) -> int:
        """Values in one cache slot (all kv heads of one token)."""
        return self.num_kv_heads * self.head_dim

    @property
    def qkv_width(self) -> int:
        """Row width of the fused q|k|v projection output."""
        return (self.num_heads + 2 * self.num_kv_heads) * self.head_dim


# Qwen3 attention shapes ("Nano-vLLM Field Guide", Step 09.5; the 8B shape has 32 q heads).
QWEN3_0_6B = AttnShape(num_heads=16, num_kv_heads=8)
QWEN3_8B = AttnShape(num_heads=32, num_kv_heads=8)


@dataclass
class Seq:
    """One scheduled sequence: its block table and which tokens this step computes.

    ``num_cached`` tokens are already in the cache; this step adds ``num_new`` tokens at
    positions ``[num_cached, num_cached + num_new)``. A decode row has ``num_new == 1``. A
    padding decode row (the graph-bucket filler) has ``num_cached == num_new == 0`` and an
    empty block table.
    """

    block_table: list
    num_cached: int
    num_new: int


@dataclass
class Step:
    """One forward step: prefill sequences and decode sequences share one store call.

    Rows of the store call are ordered prefill tokens first, then one row per decode entry
    (padding rows included), the order the mixed-step reading fixes.
    """

    prefill: list = field(default_factory=list)
    decode: list = field(default_factory=list)

    @property
    def num_prefill_tokens(self) -> int:
        return sum(s.num_new for s in self.prefill)

    @property
    def num_rows(self) -> int:
        return self.num_prefill_tokens + len(self.decode)


@dataclass
class Workload:
    name: str
    shape: AttnShape
    num_blocks: int
    owned: np.ndarray  # bool [num_blocks]: blocks that some sequence's table names
    steps: list
    seed: int
    note: str = ""


def _blocks_for(n_tokens: int, block_size: int) -> int:
    # Block reservation of the block manager: ceil(n / block_size) blocks for n tokens.
    return -(-n_tokens // block_size)


class _Pool:
    """Hands out physical block ids in the order of a random permutation."""

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.order = rng.permutation(num_blocks).astype(np.int64)
        self.next = 0
        self.owned = np.zeros(num_blocks, dtype=bool)

    def take(self, n: int) -> list:
        if self.next + n > len(self.order):
            raise ValueError("synthetic pool too small")
        ids = [int(x) for x in self.order[self.next:self.next + n]]
        self.next += n
        self.owned[ids] = True
        return ids


def _decode_step(shape, lens, pool, pad_rows=0):
    seqs = []
    for L in lens:
        L = int(L)
        seqs.append(Seq(block_table=pool.take(_blocks_for(L, shape.block_size)),
                        num_cached=L - 1, num_new=1))
    for _ in range(pad_rows):
        seqs.append(Seq(block_table=[], num_cached=0, num_new=0))
    return seqs


def config_decode_small(seed: int = 1001) -> Workload:
    """Qwen3-0.6B decode step: 4 sequences, context lengths uniform in 1..600, 2 padding rows,
    a 16-block pool assigned by a random permutation."""
    shape = QWEN3_0_6B
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 601, size=4)
    pool = _Pool(16, rng)
    step = Step(decode=_decode_step(shape, lens, pool, pad_rows=2))
    return Workload("qwen3-0.6b decode B=4+2pad L~U[1,600]", shape, 16, pool.owned, [step], seed)


def config_prefill_varlen(seed: int = 1002) -> Workload:
    """Qwen3-0.6B varlen causal prefill: 8 prompts, lengths uniform in 64..1024, empty cache,
    K/V written to a 64-block randomly permuted pool."""
    shape = QWEN3_0_6B
    rng = np.random.default_rng(seed)
    lens = rng.integers(64, 1025, size=8)
    pool = _Pool(64, rng)
    seqs = [Seq(pool.take(_blocks_for(int(L), shape.block_size)), 0, int(L)) for L in lens]
    return Workload("qwen3-0.6b varlen prefill 8 prompts L~U[64,1024]", shape, 64, pool.owned,
                    [Step(prefill=seqs)], seed)


def config_prefix_chunked(seed: int = 1003) -> Workload:
    """Qwen3-0.6B prefix-cached + chunked prefill: 16 prompts of 2048 tokens in 4 groups of 4
    sharing their first 1024 tokens (4 full blocks already cached, aliased in 4 tables); each
    suffix is computed in two 512-token chunks (positions 1024-1535, then 1536-2047). Pool of
    128 randomly permuted blocks; the whole prompt's blocks are reserved up front."""
    shape = QWEN3_0_6B
    rng = np.random.default_rng(seed)
    pool = _Pool(128, rng)
    tables = []
    for _group in range(4):
        prefix = pool.take(4)
        for _member in range(4):
            tables.append(prefix + pool.take(4))
    steps = []
    for start in (1024, 1536):
        steps.append(Step(prefill=[Seq(list(t), start, 512) for t in tables]))
    return Workload("qwen3-0.6b prefix-cached+chunked prefill 16x2048, 512-token chunks", shape,
                    128, pool.owned, steps, seed)


def config_decode_large(seed: int = 1004) -> Workload:
    """Qwen3-0.6B decode: 256 sequences, context lengths uniform in 512..4096, pool of 4608
    blocks randomly permuted."""
    shape = QWEN3_0_6B
    rng = np.random.default_rng(seed)
    lens = rng.integers(512, 4097, size=256)
    pool = _Pool(4608, rng)
    step = Step(decode=_decode_step(shape, lens, pool))
    return Workload("qwen3-0.6b decode B=256 L~U[512,4096]", shape, 4608, pool.owned, [step],
                    seed)


def config_mixed_8b(seed: int = 1005) -> Workload:
    """Qwen3-8B (32 q / 8 kv heads) mixed step: 512 decode sequences with contexts uniform in
    256..4096 plus a fresh 4 x 1024-token prefill; pool = blocks needed + 512 spare, randomly
    permuted."""
    shape = QWEN3_8B
    rng = np.random.default_rng(seed)
    dec_lens = rng.integers(256, 4097, size=512)
    pre_lens = [1024] * 4
    need = sum(_blocks_for(int(L), shape.block_size) for L in dec_lens) + \
        sum(_blocks_for(L, shape.block_size) for L in pre_lens)
    num_blocks = need + 512
    pool = _Pool(num_blocks, rng)
    prefill = [Seq(pool.take(_blocks_for(L, shape.block_size)), 0, L) for L in pre_lens]
    decode = _decode_step(shape, dec_lens, pool)
    return Workload("qwen3-8b mixed: 512 decode L~U[256,4096] + 4x1024 prefill", shape,
                    num_blocks, pool.owned, [Step(prefill=prefill, decode=decode)], seed)


def tp_share(w: Workload, tp: int) -> Workload:
    """One rank's share of a workload under tensor parallelism of degree tp ("Nano-vLLM Field
    Guide", Step 9.5: the query and kv head counts are divided by the tp size; Step 10.1: each
    rank keeps its own cache of its heads). Sequences, block tables and seed are unchanged;
    each rank's pool rows hold Hkv / tp heads."""
    s = w.shape
    if tp < 1 or s.num_heads % tp or s.num_kv_heads % tp:
        raise ValueError(f"tp={tp} must divide {s.num_heads} q heads and {s.num_kv_heads} kv heads")
    if tp == 1:
        return w
    shape = AttnShape(s.num_heads // tp, s.num_kv_heads // tp, s.head_dim, s.block_size)
    return Workload(f"{w.name} [tp={tp}: one rank's heads]", shape, w.num_blocks, w.owned,
                    w.steps, w.seed, w.note)


CONFIGS = {
    "decode_small": config_decode_small,
    "prefill_varlen": config_prefill_varlen,
    "prefix_chunked": config_prefix_chunked,
    "decode_large": config_decode_large,
    "mixed_8b": config_mixed_8b,
}


def random_workload(seed: int, shape: AttnShape, n_prefill: int = 0, n_decode: int = 0,
                    max_len: int = 700, max_cached: int = 0, pad_rows: int = 0,
                    spare_blocks: int = 3, share_prefix: bool = False) -> Workload:
    """Small ragged workload for parity sweeps.

    Prefill prompts get ``num_new`` uniform in 1..max_len and ``num_cached`` uniform in
    0..max_cached (a prefix hit or an earlier chunk). With ``share_prefix`` the prompts share
    the full blocks of the first prompt's cached prefix. Decode rows get context lengths uniform
    in 1..max_len.
    """
    bs = shape.block_size
    rng = np.random.default_rng(seed)
    p_new = rng.integers(1, max_len + 1, size=n_prefill)
    p_cached = rng.integers(0, max_cached + 1, size=n_prefill) if max_cached else \
        np.zeros(n_prefill, dtype=np.int64)
    d_lens = rng.integers(1, max_len + 1, size=n_decode)
    shared_full = 0
    if share_prefix and n_prefill:
        shared_full = int(p_cached[0]) // bs
        p_cached = np.maximum(p_cached, shared_full * bs)
    need = sum(_blocks_for(int(c + n), bs) for c, n in zip(p_cached, p_new)) + \
        sum(_blocks_for(int(L), bs) for L in d_lens) + spare_blocks
    pool = _Pool(need, rng)
    shared = pool.take(shared_full) if shared_full else []
    prefill = []
    for c, n in zip(p_cached, p_new):
        total = _blocks_for(int(c + n), bs)
        prefill.append(Seq(list(shared) + pool.take(total - len(shared)), int(c), int(n)))
    decode = _decode_step(shape, d_lens, pool, pad_rows)
    return Workload(f"random seed={seed}", shape, need, pool.owned,
                    [Step(prefill=prefill, decode=decode)], seed)


@dataclass
class StepTensors:
    """Device tensors of one step. ``value`` is a strided view into ``qkv`` (the fused
    projection output), ``key`` is contiguous, like the tensors the store receives."""

    qkv: torch.Tensor     # [N, (Hq + 2 Hkv) d] bf16
    q_prefill: torch.Tensor  # [N_prefill_tokens, Hq, d] bf16 contiguous
    q_decode: torch.Tensor   # [N_decode_rows, Hq, d] bf16 contiguous
    key: torch.Tensor     # [N, Hkv, d] bf16 contiguous
    value: torch.Tensor   # [N, Hkv, d] bf16 view, row stride (Hq + 2 Hkv) d


def _randn_bf16(shape, gen, device, chunk_rows=1 << 16):
    rows = shape[0]
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(rows, -1)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    return out


def make_cache(w: Workload, device="cpu", poison: bool = False, gen: Optional[torch.Generator] = None):
    """K and V pools, each [num_blocks * block_size, Hkv * d] bf16 (the per-layer view
    [num_blocks, block_size, Hkv, d] flattened over its first two dims)."""
    s = w.shape
    if gen is None:
        gen = torch.Generator(device=device).manual_seed(w.seed)
    n_slots = w.num_blocks * s.block_size
    k_cache = _randn_bf16((n_slots, s.row_elems), gen, device)
    v_cache = _randn_bf16((n_slots, s.row_elems), gen, device)
    if poison:
        unowned = torch.from_numpy(np.nonzero(~w.owned)[0]).to(device)
        for c in (k_cache, v_cache):
            c.view(w.num_blocks, s.block_size * s.row_elems)[unowned] = \
                torch.tensor(BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16).to(device)
    return k_cache, v_cache, gen


def make_step_tensors(w: Workload, step: Step, gen: torch.Generator, device="cpu") -> StepTensors:
    s = w.shape
    n = step.num_rows
    npre = step.num_prefill_tokens
    qkv = _randn_bf16((n, s.qkv_width), gen, device)
    qd = s.num_heads * s.head_dim
    kd = s.num_kv_heads * s.head_dim
    q_all = qkv[:, :qd].reshape(n, s.num_heads, s.head_dim)
    key = qkv[:, qd:qd + kd].contiguous().view(n, s.num_kv_heads, s.head_dim)
    value = qkv[:, qd + kd:].view(n, s.num_kv_heads, s.head_dim)
    return StepTensors(qkv=qkv, q_prefill=q_all[:npre].contiguous(),
                       q_decode=q_all[npre:].contiguous(), key=key, value=value)


def materialize(w: Workload, device="cpu", poison: bool = False):
    """Cache pools plus per-step tensors, drawn in the recipe's order."""
    k_cache, v_cache, gen = make_cache(w, device, poison)
    steps = [make_step_tensors(w, st, gen, device) for st in w.steps]
    return k_cache, v_cache, steps
