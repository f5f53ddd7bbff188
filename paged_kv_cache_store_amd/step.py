"""One forward step of the paged-KV hot path on the GPU: store, then prefill, then decode.

This is the runner-side glue ("Nano-vLLM Field Guide", Step 07.5-07.8 and Step 10.3): the
library's host metadata builder turns each step's sequence descriptions into slot mapping,
cumulative lengths, context lengths and padded block tables; they are copied to the device
once; then one store call writes every new K/V row (prefill rows first, then decode rows),
and the attention calls read through the block tables. Only marshalling happens here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import nvpaged
from .workloads import AttnShape, Step, StepTensors


@dataclass
class DeviceStep:
    shape: AttnShape
    tensors: StepTensors
    slot_mapping: torch.Tensor            # int32 [N]
    n_prefill_seqs: int
    cu_seqlens_q: Optional[torch.Tensor]  # int32 [B+1]
    cu_seqlens_k: Optional[torch.Tensor]
    max_seqlen_q: int
    max_seqlen_k: int
    prefill_tables: Optional[torch.Tensor]
    context_lens: Optional[torch.Tensor]  # int32 [B_dec]
    decode_tables: Optional[torch.Tensor]
    workspace: Optional[torch.Tensor]
    host: dict                            # the host metadata, for checks and accounting
    positions: Optional[torch.Tensor] = None  # int64 [N]: position of each row's token
    out_prefill: Optional[torch.Tensor] = None
    out_decode: Optional[torch.Tensor] = None
    counters: Optional[torch.Tensor] = None   # int32 [B_dec * Hkv], zero: one-launch decode merge


def token_positions(step: Step) -> np.ndarray:
    """Position of every row's token, prefill rows then decode rows: a prompt computes
    positions num_cached .. num_cached + num_new - 1, a decode row its last position (0 for a
    padding row)."""
    parts = [np.arange(s.num_cached, s.num_cached + s.num_new, dtype=np.int64)
             for s in step.prefill]
    parts.append(np.array([max(s.num_cached + s.num_new - 1, 0) for s in step.decode],
                          dtype=np.int64))
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def prepare_step(shape: AttnShape, step: Step, tensors: StepTensors, device) -> DeviceStep:
    bs = shape.block_size
    host = {}
    slots = []
    cu_q = cu_k = pt = cl = dt = ws = None
    mq = mk = 0
    if step.prefill:
        p = nvpaged.nv_prepare_prefill(step.prefill, bs)
        host["prefill"] = p
        slots.append(p["slot_mapping"])
        cu_q = torch.from_numpy(p["cu_seqlens_q"]).to(device)
        cu_k = torch.from_numpy(p["cu_seqlens_k"]).to(device)
        pt = torch.from_numpy(p["block_tables"]).to(device)
        mq, mk = p["max_seqlen_q"], p["max_seqlen_k"]
    if step.decode:
        d = nvpaged.nv_prepare_decode(step.decode, bs)
        host["decode"] = d
        slots.append(d["slot_mapping"])
        cl = torch.from_numpy(d["context_lens"]).to(device)
        dt = torch.from_numpy(d["block_tables"]).to(device)
        ws = nvpaged.decode_workspace(tensors.q_decode, shape.num_kv_heads, dt, bs)
    sm = np.concatenate(slots) if slots else np.zeros(0, np.int32)
    host["slot_mapping"] = sm
    host["positions"] = token_positions(step)
    ds = DeviceStep(shape, tensors, torch.from_numpy(sm).to(device), len(step.prefill), cu_q,
                    cu_k, mq, mk, pt, cl, dt, ws, host)
    ds.positions = torch.from_numpy(host["positions"]).to(device)
    if step.prefill:
        ds.out_prefill = torch.empty_like(tensors.q_prefill)
    if step.decode:
        ds.out_decode = torch.empty_like(tensors.q_decode)
        ds.counters = nvpaged.decode_counters(len(step.decode), shape.num_kv_heads, device)
    return ds


def run_store(ds: DeviceStep, k_cache, v_cache, stream=None) -> None:
    t = ds.tensors
    nvpaged.nv_store_kvcache(t.key, t.value, k_cache, v_cache, ds.slot_mapping, stream)


def run_prefill(ds: DeviceStep, k_cache, v_cache, scale: float, stream=None) -> None:
    if ds.cu_seqlens_q is None:
        return
    s = ds.shape
    nvpaged.nv_paged_attn_prefill(ds.tensors.q_prefill, k_cache, v_cache, ds.cu_seqlens_q,
                                  ds.cu_seqlens_k, ds.max_seqlen_q, ds.max_seqlen_k,
                                  ds.prefill_tables, s.num_kv_heads, s.block_size, scale,
                                  out=ds.out_prefill, stream=stream)


def run_norm_rope_store(ds: DeviceStep, k_cache, v_cache, q_norm_weight, k_norm_weight,
                        cos_sin_cache, eps: float = 1e-6, stream=None):
    """The step's rows through the fused per-head QK RMSNorm + rotary embedding + K/V store:
    returns (q [N, Hq, d], k [N, Hkv, d]) normalised and rotated (k also stored)."""
    s = ds.shape
    return nvpaged.nv_qk_norm_rope_store(ds.tensors.qkv, ds.positions, q_norm_weight,
                                         k_norm_weight, cos_sin_cache, eps, k_cache, v_cache,
                                         ds.slot_mapping, s.num_heads, s.num_kv_heads,
                                         want_k=True, stream=stream)


def run_prefill_packed(ds: DeviceStep, scale: float, stream=None) -> None:
    """Prefill over the step's own fresh K/V rows, no block table (the engine's path when no
    prompt has cached context); the prefill tokens are the step's first rows."""
    if ds.cu_seqlens_q is None:
        return
    if ds.host["prefill"]["has_cached_context"]:
        raise ValueError("packed prefill needs prompts without cached context")
    t = ds.tensors
    n = t.q_prefill.shape[0]
    nvpaged.nv_attn_prefill_packed(t.q_prefill, t.key[:n], t.value[:n], ds.cu_seqlens_q,
                                   ds.cu_seqlens_k, ds.max_seqlen_q, ds.max_seqlen_k, scale,
                                   out=ds.out_prefill, stream=stream)


def run_decode(ds: DeviceStep, k_cache, v_cache, scale: float, stream=None) -> None:
    if ds.context_lens is None:
        return
    s = ds.shape
    nvpaged.nv_paged_attn_decode(ds.tensors.q_decode, k_cache, v_cache, ds.context_lens,
                                 ds.decode_tables, s.num_kv_heads, s.block_size, scale,
                                 workspace=ds.workspace, out=ds.out_decode, stream=stream)


def run_decode_store(ds: DeviceStep, k_cache, v_cache, scale: float, stream=None) -> None:
    """A decode-only step's store and decode in one launch, split rows merged in the same
    launch (the step's rows are all decode rows, one per sequence, in the order of
    ``context_lens``)."""
    if ds.context_lens is None:
        return
    s = ds.shape
    t = ds.tensors
    nvpaged.nv_paged_attn_decode_store(t.q_decode, t.key, t.value, ds.slot_mapping, k_cache,
                                       v_cache, ds.context_lens, ds.decode_tables,
                                       s.num_kv_heads, s.block_size, scale,
                                       workspace=ds.workspace, out=ds.out_decode,
                                       counters=ds.counters, stream=stream)


def run_step(ds: DeviceStep, k_cache, v_cache, scale: Optional[float] = None, stream=None):
    """store -> prefill -> decode on one stream; returns (prefill_out, decode_out)."""
    if scale is None:
        scale = ds.shape.head_dim ** -0.5
    run_store(ds, k_cache, v_cache, stream)
    run_prefill(ds, k_cache, v_cache, scale, stream)
    run_decode(ds, k_cache, v_cache, scale, stream)
    return ds.out_prefill, ds.out_decode
