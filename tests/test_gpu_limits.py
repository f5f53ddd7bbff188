"""GPU parity at the documented size limits of the C ABI.

- Decode at the largest batch (65535 rows, two of them padding) with short contexts: the
  longest-first order over 65535 rows, a grid of half a million workgroups, and the
  allocation-free entry point's workspace at that size, all against the oracle.
- Paged prefill whose block-table prefix fills the LDS staging area exactly
  (ceil(max_seqlen_k / block_size) == 2048 entries), with whole-block tiles (block size 8:
  a 64-key tile spans 8 blocks, so every tile takes the per-key lookup) and with one-key blocks.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_store_amd import nvpaged, workloads
from paged_kv_cache_store_amd import step as gstep
from gpu_common import Run, assert_attn_close, check_metadata, check_pools_bit_exact
from helpers import bits

pytestmark = pytest.mark.gpu


def test_decode_max_batch():
    shape = workloads.AttnShape(16, 8, 128, 16)
    w = workloads.random_workload(65535, shape, 0, 65533, max_len=16, pad_rows=2)
    run = Run(w)
    print("[limits] decode of 65535 rows", flush=True)
    ds = run.gpu_step(0)
    om = run.oracle_store(0)
    check_metadata(ds, om)
    check_pools_bit_exact(run, "max batch store")
    ids, ref = run.oracle_decode(0)
    print(assert_attn_close(ds.out_decode[ids], ref, "max batch decode"))
    assert torch.count_nonzero(ds.out_decode[65533:]).item() == 0
    out = torch.full_like(ds.out_decode, float("nan"))
    nvpaged.nv_paged_attn_decode_noalloc(ds.tensors.q_decode, run.k_cache, run.v_cache,
                                         ds.context_lens, ds.decode_tables, shape.num_kv_heads,
                                         shape.block_size, run.scale, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(ds.out_decode)), "allocation-free decode differs"


@pytest.mark.parametrize("bs", [8, 1])
def test_prefill_full_table_prefix(bs):
    shape = workloads.AttnShape(16, 8, 128, bs)
    lk_max = 2048 * bs
    rng = np.random.default_rng(2048 + bs)
    pre = [(lk_max - 64, 64), (0, 100), (lk_max - 300, 17)]
    need = sum(-(-(c + n) // bs) for c, n in pre) + 2
    pool = workloads._Pool(need, rng)
    prefill = [workloads.Seq(pool.take(-(-(c + n) // bs)), c, n) for c, n in pre]
    w = workloads.Workload(f"full table prefix bs{bs}", shape, need, pool.owned,
                           [workloads.Step(prefill=prefill)], 2048 + bs)
    run = Run(w)
    ds = gstep.prepare_step(shape, w.steps[0], run.tensors[0], "cuda")
    assert -(-ds.max_seqlen_k // bs) == 2048
    print(f"[limits] prefill with a 2048-entry table prefix, block size {bs}", flush=True)
    gstep.run_step(ds, run.k_cache, run.v_cache, run.scale)
    torch.cuda.synchronize()
    om = run.oracle_store(0)
    check_pools_bit_exact(run, "full table store")
    rows, ref = run.oracle_prefill(0, om)
    print(assert_attn_close(ds.out_prefill[rows], ref, f"full table prefix bs{bs}"))


def test_empty_inputs_change_nothing():
    """Every entry point called with nothing to do (no tokens, no sequences) returns success
    and leaves its outputs and the pools untouched."""
    dev = torch.device("cuda")
    shape = workloads.QWEN3_0_6B
    D = shape.row_elems
    k = torch.randn(64, D, device=dev).bfloat16()
    v = torch.randn(64, D, device=dev).bfloat16()
    k0, v0 = bits(k).copy(), bits(v).copy()
    key = torch.empty(0, shape.num_kv_heads, shape.head_dim, dtype=torch.bfloat16, device=dev)
    slots = torch.empty(0, dtype=torch.int32, device=dev)
    nvpaged.nv_store_kvcache(key, key, k, v, slots)
    q = torch.empty(0, shape.num_heads, shape.head_dim, dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(1, dtype=torch.int32, device=dev)
    tables = torch.empty(0, 1, dtype=torch.int32, device=dev)
    out = nvpaged.nv_paged_attn_prefill(q, k, v, cu, cu, 0, 0, tables, shape.num_kv_heads,
                                        shape.block_size, 0.088)
    assert out.numel() == 0
    lens = torch.empty(0, dtype=torch.int32, device=dev)
    ws = torch.empty(1, dtype=torch.uint8, device=dev)
    nvpaged.nv_paged_attn_decode(q, k, v, lens, tables, shape.num_kv_heads, shape.block_size,
                                 0.088, workspace=ws, out=q)
    nvpaged.nv_paged_attn_decode_noalloc(q, k, v, lens, tables, shape.num_kv_heads,
                                         shape.block_size, 0.088, out=q)
    nvpaged.nv_paged_attn_decode_store(q, key, key, slots, k, v, lens, tables,
                                       shape.num_kv_heads, shape.block_size, 0.088,
                                       workspace=ws, out=q)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), k0) and np.array_equal(bits(v), v0)
