"""Decode steps replayed from HIP graphs, one graph per batch-size bucket.

Operation ("Nano-vLLM Field Guide", Step 7.9, capture_cudagraph; Step 7.8, run_model): the K/V
store and the paged decode attention of a decode step are recorded once per bucket (1, 2, 4,
8, then every multiple of 16 up to the largest batch) against static buffers sized for the
largest batch, largest bucket first, all graphs sharing one memory pool. A step of batch b
copies its inputs into the first b rows of the static buffers and replays the smallest bucket
>= b. The rows past b are padding: their slot is -1 (the store writes nothing) and their
context length 0 (the attention writes zeros and reads nothing), so padding never touches the
pool or the real rows. Block-table rows are not cleared between steps: entries past a row's
own context are never read.

The recorded launches are the library's kernels only (no memset nodes); padding values are
written by ordinary eager fills before the replay. By default (``fused=True``) each layer
records one store+decode call (nv_paged_attn_decode_store, split rows merged in the same
launch through arrival counters) instead of the store and the decode; ``fused=False``
records the two calls. Both give the same bits.
"""
from __future__ import annotations

import torch

from . import nvpaged
from .workloads import AttnShape


def buckets(max_bs: int) -> list:
    """Captured batch sizes: 1, 2, 4, 8, then multiples of 16 up to max_bs."""
    out = [b for b in (1, 2, 4, 8) if b <= max_bs]
    out += list(range(16, max_bs + 1, 16))
    if not out or out[-1] < max_bs:
        out.append(max_bs)
    return out


class DecodeGraphs:
    """Store + decode replayed from graphs, for one layer or a stack of layers. ``k_cache`` /
    ``v_cache`` are a layer's pool views (or lists of them, one per layer; the step's rows go
    to every layer); ``max_blocks`` is the block-table width (ceil of the longest context over
    the block size)."""

    def __init__(self, shape: AttnShape, k_cache, v_cache, max_bs: int, max_blocks: int,
                 scale: float | None = None, fused: bool = True,
                 merge_in_kernel: bool = True):
        if max_bs < 1 or max_blocks < 1:
            raise ValueError("max_bs and max_blocks must be positive")
        self.shape = shape
        self.fused = fused  # one store+decode launch per layer instead of two
        # fused only: split rows merged by the split kernel's last workgroup (arrival counters
        # shared by all layers and buckets; every call leaves them zero), no merge kernel
        self.merge_in_kernel = fused and merge_in_kernel
        self.k_caches = list(k_cache) if isinstance(k_cache, (list, tuple)) else [k_cache]
        self.v_caches = list(v_cache) if isinstance(v_cache, (list, tuple)) else [v_cache]
        if len(self.k_caches) != len(self.v_caches) or not self.k_caches:
            raise ValueError("one K and one V pool per layer")
        k_cache = self.k_caches[0]
        self.scale = shape.head_dim ** -0.5 if scale is None else scale
        dev = k_cache.device
        hq, hkv, d = shape.num_heads, shape.num_kv_heads, shape.head_dim
        self.max_bs = max_bs
        self.q = torch.zeros(max_bs, hq, d, dtype=torch.bfloat16, device=dev)
        self.key = torch.zeros(max_bs, hkv, d, dtype=torch.bfloat16, device=dev)
        self.value = torch.zeros(max_bs, hkv, d, dtype=torch.bfloat16, device=dev)
        self.slot_mapping = torch.full((max_bs,), -1, dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros(max_bs, dtype=torch.int32, device=dev)
        self.block_tables = torch.full((max_bs, max_blocks), -1, dtype=torch.int32, device=dev)
        self.out = torch.zeros(len(self.k_caches), max_bs, hq, d, dtype=torch.bfloat16,
                               device=dev)
        # One workspace for all buckets: the split length (and so the size) depends on the
        # batch and is not monotonic in it, so take the largest over the buckets.
        ws = max(nvpaged.nv_paged_attn_decode_workspace_size(b, hq, hkv, d, max_blocks,
                                                             shape.block_size)
                 for b in buckets(max_bs))
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.counters = (nvpaged.decode_counters(max_bs, shape.num_kv_heads, dev)
                         if self.merge_in_kernel else None)
        self.graphs = {}
        self.pool = None
        for bs in reversed(buckets(max_bs)):
            self._launch(bs)  # warm-up, eager
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, self.pool):
                self._launch(bs)
            if self.pool is None:
                self.pool = g.pool()
            self.graphs[bs] = g
            torch.cuda.synchronize()

    def _launch(self, bs: int) -> None:
        s = self.shape
        for layer, (kc, vc) in enumerate(zip(self.k_caches, self.v_caches)):
            if self.fused:
                nvpaged.nv_paged_attn_decode_store(
                    self.q[:bs], self.key[:bs], self.value[:bs], self.slot_mapping[:bs], kc, vc,
                    self.context_lens[:bs], self.block_tables[:bs], s.num_kv_heads,
                    s.block_size, self.scale, workspace=self.workspace,
                    out=self.out[layer, :bs], counters=self.counters)
                continue
            nvpaged.nv_store_kvcache(self.key[:bs], self.value[:bs], kc, vc,
                                     self.slot_mapping[:bs])
            nvpaged.nv_paged_attn_decode(self.q[:bs], kc, vc, self.context_lens[:bs],
                                         self.block_tables[:bs], s.num_kv_heads, s.block_size,
                                         self.scale, workspace=self.workspace,
                                         out=self.out[layer, :bs])

    def bucket_for(self, bs: int) -> int:
        for b in sorted(self.graphs):
            if b >= bs:
                return b
        raise ValueError(f"batch {bs} exceeds the largest captured batch {self.max_bs}")

    def _stage(self, q, key, value, slot_mapping, context_lens, block_tables) -> int:
        """Copies a step's inputs into the static buffers, padded; returns the bucket."""
        bs = q.shape[0]
        b = self.bucket_for(bs)
        w = block_tables.shape[1]
        if w > self.block_tables.shape[1]:
            raise ValueError("block table wider than the captured width")
        self.q[:bs] = q
        self.key[:bs] = key
        self.value[:bs] = value
        self.slot_mapping.fill_(-1)
        self.slot_mapping[:bs] = slot_mapping
        self.context_lens.zero_()
        self.context_lens[:bs] = context_lens
        self.block_tables[:bs, :w] = block_tables
        return b

    def run(self, q: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
            slot_mapping: torch.Tensor, context_lens: torch.Tensor,
            block_tables: torch.Tensor) -> torch.Tensor:
        """One decode step of batch q.shape[0]: stores key/value rows and returns the attention
        output [bs, Hq, d] of a single layer, or [layers, bs, Hq, d] (a view of the static
        output buffer, valid until the next call)."""
        b = self._stage(q, key, value, slot_mapping, context_lens, block_tables)
        self.graphs[b].replay()
        return self._view(q.shape[0])

    def _view(self, bs: int) -> torch.Tensor:
        return self.out[0, :bs] if len(self.k_caches) == 1 else self.out[:, :bs]

    def run_eager(self, q, key, value, slot_mapping, context_lens, block_tables) -> torch.Tensor:
        """The same step with the same padded static inputs, launched eagerly (reference)."""
        b = self._stage(q, key, value, slot_mapping, context_lens, block_tables)
        self._launch(b)
        return self._view(q.shape[0])
