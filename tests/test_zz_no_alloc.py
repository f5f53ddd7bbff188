"""The allocation-free decode (nv_paged_attn_decode_noalloc, through the C ABI) against the
decode with a caller-owned workspace (nv_paged_attn_decode): the same kernels, so the outputs
must be bitwise equal. Two calls in a row on the library's one static array, the second with a
smaller input (fewer rows and splits) over the first call's leftover contents; then the first
shape again. Also checked against the oracle once, to the attention bound.
"""
import numpy as np
import pytest
import torch

from paged_kv_cache_store_amd import nvpaged, workloads
from paged_kv_cache_store_amd import step as gstep
from gpu_common import Run, assert_attn_close
from helpers import bits

pytestmark = pytest.mark.gpu


def _decode_pair(w):
    """(noalloc output, workspace output, run, device step) of a decode-only workload."""
    run = Run(w)
    ds = gstep.prepare_step(w.shape, w.steps[0], run.tensors[0], "cuda")
    gstep.run_store(ds, run.k_cache, run.v_cache)
    s = w.shape
    t = ds.tensors
    need = nvpaged.nv_paged_attn_decode_workspace_size(t.q_decode.shape[0], s.num_heads,
                                                       s.num_kv_heads, s.head_dim,
                                                       ds.decode_tables.shape[1], s.block_size)
    assert 0 < need <= nvpaged.NV_DECODE_SCRATCH_BYTES
    print(f"[noalloc] {w.name}: {t.q_decode.shape[0]} rows, workspace {need} bytes", flush=True)
    out_na = torch.full_like(t.q_decode, float("nan"))
    nvpaged.nv_paged_attn_decode_noalloc(t.q_decode, run.k_cache, run.v_cache, ds.context_lens,
                                         ds.decode_tables, s.num_kv_heads, s.block_size,
                                         run.scale, out=out_na)
    out_ws = torch.full_like(t.q_decode, float("nan"))
    nvpaged.nv_paged_attn_decode(t.q_decode, run.k_cache, run.v_cache, ds.context_lens,
                                 ds.decode_tables, s.num_kv_heads, s.block_size, run.scale,
                                 workspace=ds.workspace, out=out_ws)
    torch.cuda.synchronize()
    return out_na, out_ws, run, ds


def test_noalloc_equals_workspace_decode_twice_then_smaller():
    big = workloads.config_decode_large()  # 256 rows in two 2048-key splits, ~4.2 MiB
    small = workloads.random_workload(77, workloads.QWEN3_0_6B, 0, 5, max_len=3000, pad_rows=1)
    for i, w in enumerate((big, small, big)):
        out_na, out_ws, run, _ = _decode_pair(w)
        assert np.array_equal(bits(out_na), bits(out_ws)), f"call {i}: outputs differ"
        if i == 1:
            run.oracle_store(0)
            ids, ref = run.oracle_decode(0)
            print(assert_attn_close(out_na[ids], ref, "noalloc decode"))
