"""Shared machinery of the GPU parity tests: run one workload step through the HIP library and
through the oracle on the same seeded inputs, and compare.

The oracle side builds its own metadata (oracle.meta), stores into its own host copy of the
pools and computes attention in double precision; nothing it uses comes from the HIP path.
"""
import numpy as np
import torch

import oracle
from oracle import meta
from paged_kv_cache_store_amd import step as gpu_step
from paged_kv_cache_store_amd import workloads
from helpers import bits

ATOL_MAX = 1e-2   # max abs error bound vs the oracle
ATOL_MEAN = 1e-3  # mean abs error bound vs the oracle


def attn_bound(ref: np.ndarray) -> np.ndarray:
    """Per-element bound: 1e-2 on the computed attention value, plus the conversion of that
    value to the bf16 output ("Nano-vLLM Field Guide", Step 12.1: the output is in the model
    dtype), which moves it by at most half a bf16 ulp of the result. The oracle is fp64 and
    not rounded, so a result within 1e-2 before rounding can land up to 1e-2 + half an ulp
    from it afterwards (half an ulp is 0.0039 for |o| in [1, 2), 0.0078 in [2, 4), 0.0156 in
    [4, 8))."""
    mag = np.maximum(np.abs(ref), 1e-30)
    half_ulp = 0.5 * 2.0 ** (np.floor(np.log2(mag)) - 7)
    return ATOL_MAX + half_ulp


def assert_attn_close(gpu: torch.Tensor, ref: np.ndarray, what: str) -> dict:
    """Checks the bound element by element and returns the error statistics, including how
    many elements exceeded 1e-2 and were accepted only through the output-rounding term
    (``allowance_used``; each test prints it)."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bad = err > attn_bound(ref)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} elements over the bound; first at "
                             f"{tuple(idx)}: gpu={g[tuple(idx)]} oracle={ref[tuple(idx)]}")
    mean = float(err.mean()) if err.size else 0.0
    assert mean <= ATOL_MEAN, f"{what}: mean abs error {mean}"
    return dict(max=float(err.max()) if err.size else 0.0, mean=mean, n=int(err.size),
                allowance_used=int((err > ATOL_MAX).sum()))


class Run:
    """A workload materialised on the GPU (poisoned unowned blocks) with its host copies."""

    def __init__(self, w: workloads.Workload, poison: bool = True):
        self.w = w
        dev = torch.device("cuda")
        self.k_cache, self.v_cache, steps = workloads.materialize(w, dev, poison=poison)
        self.k_host = bits(self.k_cache).copy()
        self.v_host = bits(self.v_cache).copy()
        self.tensors = steps
        self.scale = w.shape.head_dim ** -0.5

    def gpu_step(self, i: int):
        ds = gpu_step.prepare_step(self.w.shape, self.w.steps[i], self.tensors[i], "cuda")
        gpu_step.run_step(ds, self.k_cache, self.v_cache, self.scale)
        torch.cuda.synchronize()
        return ds

    def oracle_store(self, i: int):
        """Oracle metadata + store into the host pools (in place). Returns the metadata."""
        s = self.w.shape
        st = self.w.steps[i]
        om = {}
        slots = []
        if st.prefill:
            om["prefill"] = meta.prepare_prefill(st.prefill, s.block_size)
            slots.append(om["prefill"]["slot_mapping"])
        if st.decode:
            om["decode"] = meta.prepare_decode(st.decode, s.block_size)
            slots.append(om["decode"]["slot_mapping"])
        om["slot_mapping"] = np.concatenate(slots)
        qkv = bits(self.tensors[i].qkv)
        D = s.row_elems
        off = s.num_heads * s.head_dim
        oracle.store_kvcache(qkv[:, off:off + D], qkv[:, off + D:], self.k_host, self.v_host,
                             om["slot_mapping"])
        return om

    def oracle_prefill(self, i: int, om: dict, seq_ids=None):
        """Oracle prefill output for the chosen sequences: (rows of the packed batch, output)."""
        s = self.w.shape
        st = self.w.steps[i]
        ids = list(range(len(st.prefill))) if seq_ids is None else list(seq_ids)
        sub = [st.prefill[b] for b in ids]
        m = meta.prepare_prefill(sub, s.block_size)
        cu = om["prefill"]["cu_seqlens_q"]
        rows = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in ids])
        q = bits(self.tensors[i].q_prefill)[rows]
        out = oracle.attn_prefill(q, self.k_host, self.v_host, m["cu_seqlens_q"],
                                  m["cu_seqlens_k"], m["block_tables"], s.num_heads,
                                  s.num_kv_heads, s.head_dim, s.block_size, self.scale)
        return rows, out

    def oracle_decode(self, i: int, seq_ids=None):
        s = self.w.shape
        st = self.w.steps[i]
        ids = list(range(len(st.decode))) if seq_ids is None else list(seq_ids)
        sub = [st.decode[b] for b in ids]
        m = meta.prepare_decode(sub, s.block_size)
        bt = m["block_tables"] if m["block_tables"].shape[1] else np.full((len(ids), 1), -1,
                                                                          np.int32)
        q = bits(self.tensors[i].q_decode)[ids]
        out = oracle.attn_decode(q, self.k_host, self.v_host, m["context_lens"], bt,
                                 s.num_heads, s.num_kv_heads, s.head_dim, s.block_size,
                                 self.scale)
        return ids, out


def check_pools_bit_exact(run: Run, what: str):
    kg, vg = bits(run.k_cache), bits(run.v_cache)
    for g, h, nm in ((kg, run.k_host, "k_cache"), (vg, run.v_host, "v_cache")):
        diff = np.nonzero(np.any(g != h, axis=1))[0]
        assert diff.size == 0, f"{what}: {nm} differs in {diff.size} slots, first {diff[:5]}"


def check_metadata(ds, om: dict):
    assert np.array_equal(ds.host["slot_mapping"], om["slot_mapping"])
    if "prefill" in om:
        for k in ("cu_seqlens_q", "cu_seqlens_k"):
            assert np.array_equal(ds.host["prefill"][k], om["prefill"][k])
    if "decode" in om:
        assert np.array_equal(ds.host["decode"]["context_lens"], om["decode"]["context_lens"])
